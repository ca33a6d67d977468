// Device building blocks shared by the E8 projection kernels (gfx950, wave64).
//
// Work mapping: one lane owns one group of 8 consecutive columns (16 bytes of
// bf16 or 32 bytes of float32), so a wave covers 64 consecutive groups and a
// Walsh-Hadamard block of b <= 128 columns lives in b/8 consecutive lanes of
// one 16-lane DPP row.  Butterfly stages of stride 1, 2, 4 run inside a lane,
// strides 8..64 run across lanes.
//
// Numerics follow the contract written in include/e8q.h; every float32 step
// is a single IEEE operation (the library is built with -ffp-contract=off).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e8q.h"

namespace e8q {

constexpr int kWave = 64;
constexpr float kXLimit = 8192.0f;          // |x_i| >= 2^13 -> group treated as invalid
constexpr float kFastDecision = 0x1p-17f;   // float32 coset decision is trusted beyond this

// ------------------------------------------------------------------ division
// Unsigned 32-bit division by a runtime constant d >= 1 via a multiply-high
// (Granlund & Montgomery 1994, round-up multiplier with the add fix-up).
struct FastDiv {
    uint32_t d, m, sh1, sh2;
};

__host__ inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    f.sh1 = l < 1 ? l : 1;
    f.sh2 = l > 1 ? l - 1 : 0;
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    uint32_t t = __umulhi(n, f.m);
    return (t + ((n - t) >> f.sh1)) >> f.sh2;
}

// ------------------------------------------------------------------ loads
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Load one group (8 values) as float32.  bf16: one 16-byte load.
__device__ __forceinline__ void load_group(const uint16_t* w, uint64_t g, float (&v)[8]) {
    const uint4 p = *reinterpret_cast<const uint4*>(w + g * 8);
    v[0] = __uint_as_float(p.x << 16);
    v[1] = __uint_as_float(p.x & 0xFFFF0000u);
    v[2] = __uint_as_float(p.y << 16);
    v[3] = __uint_as_float(p.y & 0xFFFF0000u);
    v[4] = __uint_as_float(p.z << 16);
    v[5] = __uint_as_float(p.z & 0xFFFF0000u);
    v[6] = __uint_as_float(p.w << 16);
    v[7] = __uint_as_float(p.w & 0xFFFF0000u);
}

__device__ __forceinline__ void load_group(const float* w, uint64_t g, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(w + g * 8);
    const float4 b = *reinterpret_cast<const float4*>(w + g * 8 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Multiply by the per-column signs (+-1 bytes): exact.
__device__ __forceinline__ void apply_signs(const int8_t* signs, uint32_t col0, float (&v)[8]) {
    const uint2 sb = *reinterpret_cast<const uint2*>(signs + col0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t word = i < 4 ? sb.x : sb.y;
        const uint32_t neg = (word >> (8 * (i & 3) + 7)) & 1u;
        v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (neg << 31));
    }
}

// ------------------------------------------------------------------ Hadamard
// Un-normalized Sylvester WHT over blocks of HB columns held by HB/8 lanes.
// Stage order: stride 1, 2, 4 inside a lane, then strides 8, 16, 32, 64
// across lanes; each butterfly maps (p, q) to (p + q, p - q) exactly as the
// contract states.
//
// Cross-lane stages use one v_fmac_f32 with a DPP-permuted operand per
// element: new = own + eps * partner.  gfx9 DPP has no xor-4 lane pattern, so
// logical lane L of a 16-lane row sits on physical lane
// P = L0*1 ^ L1*2 ^ L2*7 ^ L3*8: logical partners L^1, L^2, L^4, L^8 are then
// the physical patterns quad_perm[1,0,3,2], quad_perm[2,3,0,1],
// row_half_mirror (xor 7) and row_ror:8 (xor 8).  With eps = +1 on the lane
// holding the lower index and -1 on the other, a lane keeps the butterfly
// result times a sign s_L = (-1)^popcount(L) (exactly: rounding to nearest
// is symmetric), which the caller folds into the row coefficient.

// Logical position of this physical lane inside its 16-lane row.
__device__ __forceinline__ uint32_t logical_lane(uint32_t lane) {
    const uint32_t p = lane & 15u;
    return p ^ (((p >> 2) & 1u) * 3u);
}

template <int HB>
__device__ __forceinline__ void fwht_inlane(float (&v)[8]) {
    if constexpr (HB >= 8) {
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if ((i & h) == 0) {
                    const float p = v[i], q = v[i + h];
                    v[i] = p + q;
                    v[i + h] = p - q;
                }
            }
        }
    }
}

#define E8Q_BFLY8(PAT, E)                                                        \
    "v_fmac_f32_dpp %0, %0, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %1, %1, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %2, %2, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %3, %3, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %4, %4, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %5, %5, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %6, %6, " E " " PAT " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %7, %7, " E " " PAT " row_mask:0xf bank_mask:0xf\n"
#define E8Q_S0 E8Q_BFLY8("quad_perm:[1,0,3,2]", "%8")
#define E8Q_S1 E8Q_BFLY8("quad_perm:[2,3,0,1]", "%9")
#define E8Q_S2 E8Q_BFLY8("row_half_mirror", "%10")
#define E8Q_S3 E8Q_BFLY8("row_ror:8", "%11")
// s_nop 4: DPP reads a VGPR that the preceding code may have just written
// (and EXEC may just have been restored); five wait states cover both.
#define E8Q_XLANE(BODY)                                                          \
    asm volatile("s_nop 4\n" BODY                                                 \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]),     \
                   "+v"(v[5]), "+v"(v[6]), "+v"(v[7])                              \
                 : "v"(eps[0]), "v"(eps[1]), "v"(eps[2]), "v"(eps[3]))

// Cross-lane stages; must run with all 64 lanes active.
template <int HB>
__device__ __forceinline__ void fwht_xlane(float (&v)[8], const float (&eps)[4]) {
    if constexpr (HB == 16) E8Q_XLANE(E8Q_S0);
    if constexpr (HB == 32) E8Q_XLANE(E8Q_S0 E8Q_S1);
    if constexpr (HB == 64) E8Q_XLANE(E8Q_S0 E8Q_S1 E8Q_S2);
    if constexpr (HB == 128) E8Q_XLANE(E8Q_S0 E8Q_S1 E8Q_S2 E8Q_S3);
}

// Per-lane constants of the cross-lane stages.
struct LaneFwht {
    float eps[4];
    uint32_t sign;      // bit 31 set when the lane holds minus the transform
    uint32_t logical;   // logical lane inside the 16-lane row
};

template <int HB>
__device__ __forceinline__ LaneFwht lane_fwht(uint32_t lane) {
    LaneFwht f;
    f.logical = logical_lane(lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) f.eps[k] = ((f.logical >> k) & 1u) ? -1.0f : 1.0f;
    const uint32_t used = HB >= 16 ? uint32_t(HB / 8 - 1) : 0u;
    f.sign = (uint32_t(__popc(f.logical & used)) & 1u) << 31;
    return f;
}

// ------------------------------------------------------------------ E8
// Nearest E8 point of x (finite, |x_i| < 2^13); writes 2z.
__device__ __forceinline__ void nearest_e8(const float (&x)[8], int (&t)[8]) {
    float a[8];
    int n[8], sg[8];
    int sum_n = 0, sum_s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float r = __builtin_rintf(x[i]);
        a[i] = fabsf(x[i] - r);
        sg[i] = x[i] >= r ? 1 : -1;
        n[i] = int(r);
        sum_n += n[i];
        sum_s += sg[i];
    }
    float amax = a[0], amin = a[0];
    int k = 0, m = 0;
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        if (a[i] > amax) { amax = a[i]; k = i; }
        if (a[i] < amin) { amin = a[i]; m = i; }
    }
    const bool odd0 = (sum_n & 1) != 0;
    const bool odd1 = ((2 * sum_n + sum_s) & 3) != 0;
    float t32 = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    t32 = t32 - 2.0f;
    if (odd0) t32 = t32 + (1.0f - 2.0f * amax);
    if (odd1) t32 = t32 - 2.0f * amin;
    bool d8;
    if (fabsf(t32) > kFastDecision) {
        d8 = t32 < 0.0f;
    } else {
        // the contract's float64 expression, same order
        double t64 = ((double(a[0]) + double(a[1])) + (double(a[2]) + double(a[3]))) +
                     ((double(a[4]) + double(a[5])) + (double(a[6]) + double(a[7])));
        t64 = t64 - 2.0;
        if (odd0) t64 = t64 + (1.0 - 2.0 * double(amax));
        if (odd1) t64 = t64 - 2.0 * double(amin);
        d8 = t64 <= 0.0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int base = 2 * n[i];
        const int fix0 = (odd0 && i == k) ? 2 * sg[i] : 0;
        const int fix1 = (odd1 && i == m) ? 2 * sg[i] : 0;
        t[i] = d8 ? base + fix0 : base + sg[i] - fix1;
    }
}

// Validity of a normalized group: all |x_i| < 2^13 (false for NaN/Inf).
// Returns 0 if valid, else the status bit to raise.
__device__ __forceinline__ uint32_t group_invalid_bits(const float (&x)[8]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) ok = ok && (fabsf(x[i]) < kXLimit);
    if (ok) return 0u;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) finite = finite && __builtin_isfinite(x[i]);
    return finite ? uint32_t(E8Q_STATUS_X_RANGE) : uint32_t(E8Q_STATUS_NONFINITE);
}

// Row coefficient c = fl32(kappa * fl32(1/s)); bad rows flagged.
__device__ __forceinline__ float row_coef(float s, float kappa, bool& bad) {
    const float inv = 1.0f / s;          // IEEE division (correctly rounded by default in HIP)
    const float c = kappa * inv;
    bad = !(s > 0.0f) || __builtin_isinf(s) || __builtin_isinf(c);
    return c;
}

// ------------------------------------------------------------------ stores
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // round to nearest even (inputs are never NaN here)
    uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
    b = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    return a | (b << 16);
}

__device__ __forceinline__ int sat_i8(int v, uint32_t& flags) {
    if (v > 127) { flags |= E8Q_STATUS_INT8_RANGE; return 127; }
    if (v < -128) { flags |= E8Q_STATUS_INT8_RANGE; return -128; }
    return v;
}

__device__ __forceinline__ uint2 pack_i8x8(const int (&t)[8], uint32_t& flags) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= (uint32_t(sat_i8(t[i], flags)) & 0xFFu) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= (uint32_t(sat_i8(t[4 + i], flags)) & 0xFFu) << (8 * i);
    return make_uint2(lo, hi);
}

// OR per-lane flags into the status word with one atomic per wave.
__device__ __forceinline__ void flush_status(uint32_t flags, uint32_t* status) {
    const uint64_t any = __ballot(flags != 0u);
    if (any) {
        uint32_t acc = flags;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc |= __shfl_xor(acc, off, 64);
        if ((__lane_id() == uint32_t(__ffsll((unsigned long long)any) - 1))) atomicOr(status, acc);
    }
}

}  // namespace e8q
