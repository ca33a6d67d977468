// e8q_ptq_init: PTQ initialization onto the fixed core -- a per-row scale
// search by the row's squared error, then the finite-core projection at the
// chosen scale, written as core indices (no escapes) and 2z.
//
// E8-QAT initializes its latent weights from a fixed E8 core before QAT
// (Figure 2(a) caption), which is why training starts with no escapes
// (Table 9).  The procedure is a reading (the pages give none):
//   * finite-core projection: the nearest E8 point when it is in C(B), else
//     the nearest point of C(B) by exhaustive search.  The search compares
//     keys x.t - ||t||^2/4 (t = 2z) evaluated in float64 in a fixed order
//     (exact products, pairwise sums, then the exact ||t||^2/4); equal keys go
//     to the lower core index.  This is the one explicit-codebook search of
//     the method, done once at initialization.
//   * scale search: s_k = fl32(alpha_k * s0_r) for the given multipliers; the
//     row error is the exact rational E_k = sum_i (kappa v_i - s_k t_i/2)^2;
//     the smallest error wins, NaN counts as +inf, ties go to the smaller k,
//     a candidate with an invalid scale (the projection's bad-row rule) has
//     error +inf.
//
// Exact choice by a float64 screen.  Each candidate's error is first summed in
// float64: kappa v_i and s_k t_i/2 are exact products, so every term carries
// two roundings (the difference and its square) and a sum of n non-negative
// terms in any order stays within gamma_{n+2} = (n+2)u/(1-(n+2)u) of E_k
// (u = 2^-53).  With cols <= 52216 that is below 6e-12, so a candidate whose
// float64 error is below the best's by the factor 1 + 2^-32 is certainly
// better, one above it by that factor certainly worse.  Anything in between is
// decided exactly: E_k - E_j = sum_i (c_ki^2 - 2 a_i c_ki) 2^(..)
// - (same for j), with a_i = 2 kappa v_i and c_ki = s_k t_ki as integers times
// powers of two (the a_i^2 terms are equal and cancel), summed without
// rounding into a 1024-bit fixed-point accumulator in LDS (32 limbs of 32 bits
// held in 64-bit words, so that carries wait until the end).  err_out holds
// the float64 errors, within gamma_{cols+2} of the exact ones.
//
// One block of four waves per row.  The un-normalized transform v of the
// weights is computed once (e8q_rotate.hpp) into the workspace.  Per
// candidate, the threads stride over the row's groups: the nearest E8 point
// and, for points inside the core, the group error go to LDS; groups outside
// the core are queued and searched 32 per wave at a time.  The search is a dense contraction (every
// group against every core point), so it runs on the matrix cores: the core
// points, sorted into norm shells and tiles of 32, meet a bfloat16 hi + mid
// split of the groups in one 32x32x16 MFMA per tile, which screens the
// float64 keys to within a bound; only the best tile's 32 points (and, on a
// near tie, the other tiles within the bound) are then evaluated exactly.  The
// row error is then summed from LDS.
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"
#include "e8q_rotate.hpp"

namespace e8q {

constexpr int kPtqWaves = 4;   // waves per block; one block per row
constexpr uint32_t kPtqThreads = kPtqWaves * kWave;

// Exact comparison of two candidates' errors: value = sum_i acc[i] 2^(32 i - kAccBase).
// Every term is an integer times 2^p with p >= -446 (products of float32
// values, each a multiple of 2^-149) and below 2^262 (|v| < 2^128, kappa <= 1,
// |t| <= 12); with the bit offset of a term below 2^31 and at most 2^18 terms
// per limb, no 64-bit limb overflows and the total fits the 1024 bits.
constexpr int kAccLimbs = 32;
constexpr int kAccBase = 608;
constexpr double kScreenFactor = 1.0 + 0x1p-32;   // > (1 + gamma)/(1 - gamma), gamma = gamma_{cols+2}
enum PassMode { kScreen = 0, kWrite = 1, kExact = 2 };

struct PtqArgs {
    const float* v;            // [rows_total, cols] un-normalized rotated weights
    const float* s0;
    const float* alphas;
    int32_t n_alpha;
    uint32_t rows_total;
    uint32_t cols;
    uint32_t gpr;
    float kappa;
    int core_bound;
    const double* pts64;       // [npts][9]
    uint32_t npts;
    const uint8_t* tiles;      // shell tiles (matrix-core search)
    uint32_t ntiles;
    float tmax;                // largest |t_i| of a core point (bound)
    float nmax4;               // B / 4
    float big;                 // above every approximate key (3e38)
    const uint16_t* tab;
    RankParams rp;
    float* scale_out;
    int32_t* choice_out;
    double* err_out;           // [rows_total, n_alpha] or null
    uint16_t* core_idx;
    int8_t* two_z;
    uint32_t* status;
};

__device__ __forceinline__ double group_error(const float (&v)[8], const int (&t)[8], double k64, double s64) {
    double q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double d = k64 * double(v[i]) - s64 * (0.5 * double(t[i]));
        q[i] = d * d;
    }
    return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
}

__device__ __forceinline__ void load_v(const float* row, uint32_t g, float (&v)[8]) {
    const float4* p = reinterpret_cast<const float4*>(row + uint64_t(g) * 8);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(4))) double* const_dptr;
typedef const __attribute__((address_space(4))) float* const_fptr;

// Round-to-nearest-even to bfloat16 (finite inputs), returned as float.
__device__ __forceinline__ float bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// Largest of the 16 magnitudes |d_i| (a row holds t, and -t has dot product
// -d: |d| screens the better of the two).  max(a, b) is taken as med3(a, b,
// big) with big > every value (a kernel argument, so that it is not folded
// back into a plain max, which would quiet NaNs of the raw MFMA results
// first).
__device__ __forceinline__ float tile_max(const f32x16_t& d, float big) {
    float m = __builtin_amdgcn_fmed3f(fabsf(d[0]), fabsf(d[1]), big);
    m = fmaxf(fmaxf(m, fabsf(d[2])), fabsf(d[3]));
    m = fmaxf(fmaxf(m, fabsf(d[4])), fabsf(d[5]));
    m = fmaxf(fmaxf(m, fabsf(d[6])), fabsf(d[7]));
    m = fmaxf(fmaxf(m, fabsf(d[8])), fabsf(d[9]));
    m = fmaxf(fmaxf(m, fabsf(d[10])), fabsf(d[11]));
    m = fmaxf(fmaxf(m, fabsf(d[12])), fabsf(d[13]));
    return fmaxf(fmaxf(m, fabsf(d[14])), fabsf(d[15]));
}

// Exact float64 keys of this lane's 16 rows of a tile (rows 8j + 4 half + q,
// j, q < 4: the rows an MFMA result holds for lane half `half`), each for t
// and for -t: with S the oracle's pairwise sum of x_i t_i, the key of -t is
// exactly -S - ||t||^2/4 (negation commutes with rounding).  The largest key
// wins, ties to the lower core index.  Every real row of a tile has the
// tile's norm; a pad row (t = 0, the origin's index) gets key -||t||^2/4 of
// its tile, which never reaches the best key unless the tile is the origin's
// own (where it is the origin's exact key).
__device__ __forceinline__ void eval_rows(const PtqArgs& a, const double (&x64)[8], uint32_t tile, uint32_t half,
                                          double& best, uint32_t& bi) {
    const uint4* t8 = reinterpret_cast<const uint4*>(a.tiles + size_t(a.ntiles) * 512) + size_t(tile) * 16 + 2 * half;
    const uint2* ip = reinterpret_cast<const uint2*>(a.tiles + size_t(a.ntiles) * 768) + size_t(tile) * 8 + half;
    const uint2* in = reinterpret_cast<const uint2*>(a.tiles + size_t(a.ntiles) * 832) + size_t(tile) * 8 + half;
    const double n4 = double(reinterpret_cast<const float*>(a.tiles + size_t(a.ntiles) * 896)[tile]);
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
        // a run of four consecutive rows, loaded before any is used
        const uint4 w0 = t8[4 * j], w1 = t8[4 * j + 1];
        const uint2 idp = ip[2 * j], idn = in[2 * j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 ww = (q >> 1) ? w1 : w0;
            const uint32_t lo = (q & 1) ? ww.z : ww.x, hi = (q & 1) ? ww.w : ww.y;
            double p[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = x64[i] * double(int(int8_t(lo >> (8 * i))));
                p[4 + i] = x64[4 + i] * double(int(int8_t(hi >> (8 * i))));
            }
            const double sum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            // the better of t (key sum - n4) and -t (key -sum - n4): |sum| - n4,
            // from t if sum > 0, from -t if sum < 0, the lower index if sum = 0
            const double key = fabs(sum) - n4;
            const uint32_t sh = 16u * uint32_t(q & 1);
            const uint32_t xp = (((q >> 1) ? idp.y : idp.x) >> sh) & 0xFFFFu;
            const uint32_t xn = (((q >> 1) ? idn.y : idn.x) >> sh) & 0xFFFFu;
            const uint32_t idx = sum > 0.0 ? xp : sum < 0.0 ? xn : min(xp, xn);
            const bool better = key > best || (key == best && idx < bi);
            best = better ? key : best;
            bi = better ? idx : bi;
        }
    }
}

// Matrix-core screening of one group per lane pair (lanes l and l + 32 hold
// the group of column l % 32).  x = v*c is split as x = hi + mid + r with hi,
// mid bfloat16; one 32x32x16 MFMA per tile of 32 core points computes
// t.hi + t.mid for every (point, group) pair, lanes < 32 feeding hi and lanes
// >= 32 mid against the same points.  The tiles hold one point of each pair
// +-t, so |t.x| - ||t||^2/4 screens both.  Each lane keeps, over the tiles,
// the largest approximate key of its 16 rows (M1, in tile T1) and the largest
// of the other tiles (M2).  The approximate keys are within eps of the float64
// keys:
//   eps = tmax * sum|r_i| + 2^-18 * (tmax * sum|x_i| + B/4)
// (|t_i| <= tmax; the products are exact in float32 and the sum of 16
// products plus the norm takes fewer than 2^5 roundings of at most 2^-23
// relative each).  A point whose approximate key is below best - 3 eps has a
// float64 key below that of the best tile's best point, so only tiles within
// 3 eps of the best can hold the winner.  The two lanes evaluate the best
// tile's 32 rows (64 points) exactly; if another tile comes within 3 eps (a near tie), a
// second sweep evaluates every such tile too.  The largest float64 key wins,
// ties to the lower core index.
__device__ __forceinline__ uint32_t screen_group(const PtqArgs& a, const float (&v)[8], float c, uint32_t lane) {
    const bool lo_half = lane < 32u;
    float x[8];
    bf16x8_t b;
    float rsum = 0.0f, xsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[i] = v[i] * c;
        const float hi = bf16_rne(x[i]);
        const float d = x[i] - hi;          // exact
        const float mid = bf16_rne(d);
        rsum += fabsf(d - mid);             // d - mid exact
        xsum += fabsf(x[i]);
        const uint16_t bits = uint16_t(__float_as_uint(lo_half ? hi : mid) >> 16);
        b[i] = __builtin_bit_cast(__bf16, bits);
    }
    const float eps = 1.01f * (a.tmax * rsum + 0x1p-18f * (a.tmax * xsum + a.nmax4)) + 1e-30f;

    const bf16x8_t* at = reinterpret_cast<const bf16x8_t*>(a.tiles) + (lane & 31u);
    const const_fptr n4t = (const_fptr)(uintptr_t)(a.tiles + size_t(a.ntiles) * 896);
    const f32x16_t zero = {};
    const uint32_t last = a.ntiles - 1u;
    float m1 = -__builtin_inff(), m2 = -__builtin_inff();
    uint32_t t1 = 0;
    // two tiles per step (the tile count is even), the next two tiles'
    // points loaded ahead (clamped to the last tile at the end)
    bf16x8_t p0 = at[0], p1 = at[kTileRows];
    for (uint32_t tile = 0; tile < a.ntiles; tile += 2) {
        const f32x16_t d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p0, b, zero, 0, 0, 0);
        const f32x16_t d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p1, b, zero, 0, 0, 0);
        p0 = at[size_t(min(tile + 2u, last - 1u)) * kTileRows];
        p1 = at[size_t(min(tile + 3u, last)) * kTileRows];
        // keep the loads of the next step ahead of this step's reductions
        __builtin_amdgcn_sched_barrier(0);
        const float k0 = tile_max(d0, a.big) - n4t[tile];
        const float k1 = tile_max(d1, a.big) - n4t[tile + 1u];
        m2 = __builtin_amdgcn_fmed3f(m1, m2, k0);
        t1 = k0 > m1 ? tile : t1;
        m1 = __builtin_amdgcn_fmed3f(m1, k0, a.big);
        m2 = __builtin_amdgcn_fmed3f(m1, m2, k1);
        t1 = k1 > m1 ? tile + 1u : t1;
        m1 = __builtin_amdgcn_fmed3f(m1, k1, a.big);
    }
    // combine the two halves of the tile rows (values of half 0 first)
    const float om1 = __shfl_xor(m1, 32, 64), om2 = __shfl_xor(m2, 32, 64);
    const uint32_t ot1 = uint32_t(__shfl_xor(int(t1), 32, 64));
    const float a1 = lo_half ? m1 : om1, a2 = lo_half ? m2 : om2;
    const float b1 = lo_half ? om1 : m1, b2 = lo_half ? om2 : m2;
    const uint32_t ta = lo_half ? t1 : ot1, tb = lo_half ? ot1 : t1;
    const uint32_t ts = a1 >= b1 ? ta : tb;
    const float top = fmaxf(a1, b1);
    const float comp = fmaxf(ta == ts ? a2 : a1, tb == ts ? b2 : b1);
    const bool amb = !(top - comp > 3.0f * eps);

    double x64[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x64[i] = double(x[i]);
    const uint32_t half = lane >> 5;
    double best = -__builtin_inf();
    uint32_t bi = 0xFFFFFFFFu;
    eval_rows(a, x64, ts, half, best, bi);
    // near ties between tiles: a second sweep evaluates exactly every other
    // tile whose approximate key comes within 3 eps of the best
    if (__ballot(amb)) {
        const float thr = top - 3.0f * eps;
        for (uint32_t tile = 0; tile < a.ntiles; ++tile) {
            const f32x16_t d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at[size_t(tile) * kTileRows], b, zero, 0, 0, 0);
            const float k = tile_max(d, a.big) - n4t[tile];
            if (amb && tile != ts && k >= thr) eval_rows(a, x64, tile, half, best, bi);
        }
    }
    const double ob = __shfl_xor(best, 32, 64);
    const uint32_t oi = uint32_t(__shfl_xor(int(bi), 32, 64));
    if (ob > best || (ob == best && oi < bi)) bi = oi;
    return bi;
}

// A finite float32 as m * 2^e with m an integer, |m| < 2^24, e >= -149.
__device__ __forceinline__ void f32_parts(float f, int64_t& m, int& e) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t ex = (u >> 23) & 0xFFu;
    const int64_t mag = int64_t(ex ? ((u & 0x7FFFFFu) | 0x800000u) : (u & 0x7FFFFFu));
    e = ex ? int(ex) - 150 : -149;
    m = (u >> 31) ? -mag : mag;
}

// acc += y * 2^p (|y| < 2^96, y * 2^(p mod 32) held in 128 bits), split
// over four limbs: three unsigned 32-bit chunks and a signed top.
__device__ __forceinline__ void acc_add(unsigned long long* acc, __int128 y, int p) {
    const int pos = p + kAccBase;
    const int l = pos >> 5;
    const unsigned __int128 z = static_cast<unsigned __int128>(y) << (pos & 31);
    const __int128 zs = static_cast<__int128>(z);
    atomicAdd(acc + l, (unsigned long long)uint32_t(z));
    atomicAdd(acc + l + 1, (unsigned long long)uint32_t(z >> 32));
    atomicAdd(acc + l + 2, (unsigned long long)uint32_t(z >> 64));
    atomicAdd(acc + l + 3, (unsigned long long)int64_t(zs >> 96));
}

// What one pass over a row needs besides the arguments.
struct PassCtx {
    double k64, s64;          // kappa and the candidate scale
    double* s_e;              // [gpr] group errors (screen and write passes)
    unsigned long long* acc;  // exact accumulator (exact passes)
    int64_t mk, ms;           // kappa = mk 2^ek, s = ms 2^es
    int ek, es;
    int sign;                 // +1 or -1: the candidate's side of the difference
};

// Exact pass: adds sign * sum_i (c_i^2 - 2 a_i c_i) for the group, with
// a_i = 2 kappa v_i = (mk m_i) 2^(ek + e_i + 1), c_i = s t_i = (ms t_i) 2^es.
__device__ __forceinline__ void exact_group(const PassCtx& cx, const float (&v)[8], const int (&t)[8]) {
#pragma unroll 1
    for (int i = 0; i < 8; ++i) {
        if (t[i] == 0) continue;
        int64_t mv;
        int ev;
        f32_parts(v[i], mv, ev);
        const __int128 ai = __int128(cx.mk * mv);               // |a| < 2^48
        const __int128 ci = __int128(cx.ms * int64_t(t[i]));   // |c| < 2^27
        acc_add(cx.acc, cx.sign * ci * ci, 2 * cx.es);
        acc_add(cx.acc, -cx.sign * ai * ci, cx.ek + ev + cx.es + 2);
    }
}

// The group's result for point t (core index idx): its float64 error, its
// stored point (write pass) or its exact terms (exact pass).
template <int MODE>
__device__ __forceinline__ void group_done(const PtqArgs& a, const PassCtx& cx, const float (&v)[8], const int (&t)[8],
                                           uint32_t idx, uint32_t g, uint64_t gbase) {
    if constexpr (MODE == kExact) {
        exact_group(cx, v, t);
    } else {
        cx.s_e[g] = group_error(v, t, cx.k64, cx.s64);
        if constexpr (MODE == kWrite) {
            uint32_t f8 = 0;
            *reinterpret_cast<uint2*>(a.two_z + (gbase + g) * 8) = pack_i8x8(t, f8);
            a.core_idx[gbase + g] = uint16_t(idx);
        }
    }
}

// One candidate scale over one row.  Screen and write passes return the
// float64 row error (valid on every lane; the write pass also stores the
// points); an exact pass adds its terms to cx.acc and returns 0.
template <int MODE>
__device__ double row_pass(const PtqArgs& a, uint32_t row, float c, const PassCtx& cx, uint16_t* s_list,
                           uint32_t* s_cnt, uint32_t& flags) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
    const float* vrow = a.v + uint64_t(row) * a.cols;
    const uint64_t gbase = uint64_t(row) * a.gpr;
    for (uint32_t g0 = 0; g0 < a.gpr; g0 += kPtqThreads) {
        const uint32_t g = g0 + tid;
        bool outside = false;
        if (g < a.gpr) {
            float v[8], x[8];
            load_v(vrow, g, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = v[i] * c;
            int t[8];
            const uint32_t inv = group_invalid_bits(x);
            if (inv) {
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = 0;
                if (MODE == kWrite) flags |= inv;
            } else {
                nearest_e8(x, t);
            }
            outside = norm_u32(t) > uint32_t(a.core_bound);
            if (!outside) {
                const uint32_t idx = MODE == kWrite ? core_rank(t, a.tab, a.rp) : 0u;
                group_done<MODE>(a, cx, v, t, idx, g, gbase);
            }
        }
        // the list is a work queue: its order does not affect any result
        const uint64_t m = __ballot(outside);
        uint32_t base = 0;
        if (lane == 0 && m) base = atomicAdd(s_cnt, uint32_t(__popcll(m)));
        base = __shfl(base, 0, 64);
        if (outside) s_list[base + __popcll(m & ((1ull << lane) - 1ull))] = uint16_t(g);
    }
    __syncthreads();
    const uint32_t nlist = *s_cnt;
    // groups outside the core, 32 per wave at a time (lanes l and l + 32 share one)
    for (uint32_t j0 = wv * kTileRows; j0 < nlist; j0 += kPtqWaves * kTileRows) {
        const uint32_t jn = j0 + (lane & 31u);
        const bool act = jn < nlist;
        const uint32_t g = uint32_t(s_list[act ? jn : j0]);
        float v[8];
        load_v(vrow, g, v);
        const uint32_t bi = screen_group(a, v, c, lane);
        if (act && lane < 32u) {
            const double* tp = a.pts64 + uint64_t(bi) * 9;
            int t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = int(tp[i]);
            group_done<MODE>(a, cx, v, t, bi, g, gbase);
        }
    }
    __syncthreads();
    if (tid == 0) *s_cnt = 0;
    double acc = 0.0;
    if constexpr (MODE != kExact) {
        // the row error (every wave computes the same value)
        for (uint32_t g = lane; g < a.gpr; g += kWave) acc = acc + cx.s_e[g];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
    }
    __syncthreads();   // the buffers are reused by the next pass
    return acc;
}

__device__ __forceinline__ PassCtx make_ctx(const PtqArgs& a, float s, double* s_e, unsigned long long* acc,
                                            int sign) {
    PassCtx cx;
    cx.k64 = double(a.kappa);
    cx.s64 = double(s);
    cx.s_e = s_e;
    cx.acc = acc;
    f32_parts(a.kappa, cx.mk, cx.ek);
    f32_parts(s, cx.ms, cx.es);
    cx.sign = sign;
    return cx;
}

// Exact sign of E_k - E_j for two candidates with valid scales: -1, 0 or +1
// (the same on every thread).
__device__ int exact_compare(const PtqArgs& a, uint32_t row, float sk, float ck, float sj, float cj,
                             double* s_e, unsigned long long* acc, uint16_t* s_list, uint32_t* s_cnt,
                             int* s_sign) {
    const uint32_t tid = threadIdx.x;
    if (tid < uint32_t(kAccLimbs)) acc[tid] = 0ull;
    __syncthreads();
    uint32_t dummy = 0;
    (void)row_pass<kExact>(a, row, ck, make_ctx(a, sk, s_e, acc, 1), s_list, s_cnt, dummy);
    (void)row_pass<kExact>(a, row, cj, make_ctx(a, sj, s_e, acc, -1), s_list, s_cnt, dummy);
    if (tid == 0) {
        // carries: value = sum_i d_i 2^(32 i) + top 2^1024 with 0 <= d_i < 2^32
        int64_t carry = 0;
        bool nonzero = false;
        for (int i = 0; i < kAccLimbs; ++i) {
            const int64_t x = int64_t(acc[i]) + carry;
            nonzero = nonzero || uint32_t(x) != 0u;
            carry = x >> 32;
        }
        *s_sign = carry < 0 ? -1 : (carry > 0 || nonzero) ? 1 : 0;
    }
    __syncthreads();
    const int sg = *s_sign;
    __syncthreads();
    return sg;
}

__global__ __launch_bounds__(kPtqThreads, 4) void ptq_kernel(PtqArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t tid = threadIdx.x;
    const uint32_t row = blockIdx.x;
    unsigned long long* acc = reinterpret_cast<unsigned long long*>(s_dyn);
    double* s_e = reinterpret_cast<double*>(acc + kAccLimbs);
    uint32_t* s_cnt = reinterpret_cast<uint32_t*>(s_e + a.gpr);
    int* s_sign = reinterpret_cast<int*>(s_cnt + 1);
    uint16_t* s_list = reinterpret_cast<uint16_t*>(s_sign + 1);
    if (tid == 0) *s_cnt = 0;
    __syncthreads();
    const float s0 = a.s0[row];
    uint32_t flags = 0;
    double best = __builtin_inf();
    int32_t kbest = 0;
    for (int32_t k = 0; k < a.n_alpha; ++k) {
        const float s = a.alphas[k] * s0;
        bool bad;
        const float c = row_coef(s, a.kappa, bad);
        double e = __builtin_inf();
        if (!bad) e = row_pass<kScreen>(a, row, c, make_ctx(a, s, s_e, acc, 1), s_list, s_cnt, flags);
        if (a.err_out && tid == 0) a.err_out[uint64_t(row) * uint32_t(a.n_alpha) + uint32_t(k)] = e;
        const double key = e != e ? __builtin_inf() : e;
        // key and best are the same on every thread, so every branch is uniform
        bool take;
        if (k == 0) {
            take = true;
        } else if (key == __builtin_inf()) {
            take = false;                  // cannot beat anything; equal +inf keeps the smaller k
        } else if (best == __builtin_inf()) {
            take = true;
        } else if (key * kScreenFactor < best) {
            take = true;
        } else if (best * kScreenFactor < key) {
            take = false;
        } else {
            const float sb = a.alphas[kbest] * s0;
            bool bad_b;
            const float cb = row_coef(sb, a.kappa, bad_b);
            take = exact_compare(a, row, s, c, sb, cb, s_e, acc, s_list, s_cnt, s_sign) < 0;
        }
        if (take) {
            best = key;
            kbest = k;
        }
    }
    const float s = a.alphas[kbest] * s0;
    bool bad;
    const float c = row_coef(s, a.kappa, bad);
    if (bad) {
        // the projection's bad-row rule: every point is 0
        const int t0[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const uint16_t zero_idx = uint16_t(core_rank(t0, a.tab, a.rp));
        for (uint32_t g = tid; g < a.gpr; g += kPtqThreads) {
            *reinterpret_cast<uint2*>(a.two_z + (uint64_t(row) * a.gpr + g) * 8) = make_uint2(0u, 0u);
            a.core_idx[uint64_t(row) * a.gpr + g] = zero_idx;
        }
        flags |= E8Q_STATUS_BAD_SCALE;
    } else {
        (void)row_pass<kWrite>(a, row, c, make_ctx(a, s, s_e, acc, 1), s_list, s_cnt, flags);
    }
    if (tid == 0) {
        a.scale_out[row] = s;
        if (a.choice_out) a.choice_out[row] = kbest;
    }
    flush_status(flags, a.status);
}

static size_t ptq_ws_bytes(int64_t batch, int64_t rows, int64_t cols) {
    return (size_t(batch) * size_t(rows) * size_t(cols) * 4 + 255) & ~size_t(255);
}

}  // namespace e8q

extern "C" size_t e8q_ptq_workspace_size(int64_t batch, int64_t rows, int64_t cols) {
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 8) return 0;
    return e8q::ptq_ws_bytes(batch, rows, cols);
}

extern "C" e8q_status_t e8q_ptq_init(const void* w, e8q_dtype_t w_dtype, int64_t batch, int64_t rows, int64_t cols,
                                     const float* base_scale, const float* alphas, int32_t n_alpha,
                                     const int8_t* signs, int32_t had_block, int32_t core_bound, float* scale_out,
                                     int32_t* choice_out, double* err_out, uint16_t* core_idx_out,
                                     int8_t* two_z_out, void* workspace, size_t workspace_bytes,
                                     uint32_t* status_dev, void* stream) {
    using namespace e8q;
    e8q_status_t st = check_shape(w, w_dtype, batch, rows, cols, base_scale, status_dev);
    if (st != E8Q_OK) return st;
    if (!alphas || n_alpha <= 0 || !scale_out || !core_idx_out || !two_z_out || !workspace)
        return E8Q_ERR_INVALID;
    if (core_bound < 0 || core_bound > 40) return E8Q_ERR_INVALID;
    if (signs) {
        st = check_block(signs, had_block, cols);
        if (st != E8Q_OK) return st;
    }
    if (workspace_bytes < ptq_ws_bytes(batch, rows, cols) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return E8Q_ERR_INVALID;
    const uint64_t rows_total = uint64_t(batch) * uint64_t(rows);
    const uint32_t gpr = uint32_t(cols / 8);
    const size_t lds = size_t(kAccLimbs) * 8 + size_t(gpr) * (8 + 2) + 8;
    if (lds > 64 * 1024 || rows_total >= (uint64_t(1) << 31)) return E8Q_ERR_UNSUPPORTED;
    const int hb = signs ? had_block : 0;
    const size_t rot_lds = (hb > 0 ? size_t(cols / 2) * 4 : 0) + (hb > 128 ? size_t(8 * kBlock) * 4 : 0);
    if (rot_lds > 60 * 1024) return E8Q_ERR_UNSUPPORTED;

    e8q_status_t err = E8Q_OK;
    const DevTable* tab = get_table(core_bound, err);
    if (!tab) return err;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    float* v = static_cast<float*>(workspace);
    RotArgs ra;
    ra.x = w;
    ra.xt = v;
    ra.xb = nullptr;
    ra.signs = signs;
    ra.kappa = 1.0f;                      // the un-normalized transform
    ra.cols = uint32_t(cols);
    ra.gpr = gpr;
    ra.groups = uint32_t(rows_total * gpr);
    ra.gpr_div = make_fastdiv(gpr);
    ra.num_tiles = uint32_t((uint64_t(ra.groups) + kTileGroups - 1) / kTileGroups);
    if (w_dtype == E8Q_BF16)
        launch_rotate<uint16_t>(hb, ra, rot_lds, s);
    else
        launch_rotate<float>(hb, ra, rot_lds, s);

    PtqArgs a;
    a.v = v;
    a.s0 = base_scale;
    a.alphas = alphas;
    a.n_alpha = n_alpha;
    a.rows_total = uint32_t(rows_total);
    a.cols = uint32_t(cols);
    a.gpr = gpr;
    a.kappa = kappa_for(hb);
    a.core_bound = core_bound;
    a.pts64 = tab->dpts64;
    a.npts = uint32_t(tab->size);
    a.tiles = tab->dtiles;
    a.ntiles = tab->ntiles;
    a.tmax = floorf(sqrtf(float(core_bound)));
    a.nmax4 = float(core_bound) / 4.0f;
    a.big = 3.0e38f;
    a.tab = tab->dptr;
    a.rp = tab->p;
    a.scale_out = scale_out;
    a.choice_out = choice_out;
    a.err_out = err_out;
    a.core_idx = core_idx_out;
    a.two_z = two_z_out;
    a.status = status_dev;
    launch(ptq_kernel, dim3(unsigned(rows_total)), dim3(kPtqThreads), lds, s, a);
    return launch_status();
}
