// e8q_project / e8q_project_hadamard: the QAT forward projection.
//
// E8-QAT maps every group of eight normalized weights to its nearest E8 point
// by arithmetic in every training forward pass (abstract; Figure 1(c) and
// Figure 2(b) captions), after a Hadamard transform and with reconstruction
// scales that the overview figure leaves out (Figure 2 caption).
//
// A streaming map over tiles of 4096 groups (512-thread blocks, 8 groups per
// thread, loads two groups ahead).  Rotation and the nearest point are the
// shared per-group pipeline (e8q_point.hpp); the fast path writes q = s z
// straight from the packed 2z + 64 bytes: q_i = fma(byte_i, s/2, -32 s), which
// is the single rounding of the exact product s z_i.
//
// e8q_sgd_project_hadamard fuses a QAT step's update with the next forward:
// each lane first applies the identity STE with SGD to its group of bf16
// latents (w <- bf16(fl32(w) - fl32(lr g)), NaN -> 0x7FC0, exactly as
// e8q_ste_backward), stores the new latents in place, and projects them: the
// latents are read once instead of twice per training step.
//
// e8q_sgd_project_hadamard_restore does the same before the restored
// projection below, and e8q_sgd_rotated_project_hadamard first takes a
// rotated-basis gradient back through the rotation on the same lanes
// (sigma * fl32(kappa_b H_b g), as e8q_ste_backward_hadamard) and steps the
// latents with that float32 gradient.
//
// e8q_project_hadamard_restore writes the projection back in the original
// basis instead: w_hat = sigma * fl32(T * c2), T = H_b (2z) with float32
// butterflies in the forward stage order, c2 = fl32(fl32(s kappa_b) / 2).  The
// inverse transform runs on the same lanes as the forward one (the rotation is
// orthogonal and H_b symmetric, so it is the same butterfly network followed
// by the sign flip).  On the fast path 2z + 64 is transformed instead: its
// three in-lane stages are exact and leave the offset only in element 0 (as
// 8 * 64), which is removed before the cross-lane stages.
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"

namespace e8q {

struct ProjectArgs {
    const void* w;
    uint32_t groups;
    uint32_t gpr;             // groups per row
    FastDiv gpr_div;
    FastDiv gpb_div;          // groups per batch item
    const float* scale;
    const int8_t* signs;
    uint32_t cols;
    float kappa;
    void* q;
    int q_bf16;
    int8_t* two_z;
    float* rotated;
    int core_bound;
    unsigned long long* esc;
    uint32_t* status;
    uint32_t num_tiles;
    void* w_hat;              // restored weights (original basis), or null
    int w_hat_bf16;
    const void* grad;         // SGD: bf16 gradient of the latents (same layout as w)
    float lr;
};

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    // v_cvt_pk_bf16_f32: round to nearest even (q is never NaN)
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t f = {lo, hi};
    const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

// 2z + 64 bytes -> signed 2z bytes (values are within [-64, 63])
__device__ __forceinline__ uint32_t unbias_i8x4(uint32_t t) {
    const uint32_t x = t ^ 0x40404040u;
    return x | ((x & 0x40404040u) << 1);
}

// SGD on one word of two bf16 latents; `nan` is set when a result is NaN
// (the caller then redoes the group with the scalar rule).
__device__ __forceinline__ uint32_t sgd_word(uint32_t w2, uint32_t g2, float lr, bool& nan) {
    const float w0 = __uint_as_float(w2 << 16), w1 = __uint_as_float(w2 & 0xFFFF0000u);
    const float g0 = __uint_as_float(g2 << 16), g1 = __uint_as_float(g2 & 0xFFFF0000u);
    const float n0 = w0 - lr * g0;
    const float n1 = w1 - lr * g1;
    nan = nan || (n0 != n0) || (n1 != n1);
    return bf16x2_rne(n0, n1);
}

__device__ __forceinline__ uint32_t sgd_bf16_scalar(uint32_t w, uint32_t g, float lr) {
    const float n = __uint_as_float(w << 16) - lr * __uint_as_float(g << 16);
    const uint32_t u = __float_as_uint(n);
    return n != n ? 0x7FC0u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The identity STE with SGD on one group of bf16 latents.
__device__ __forceinline__ uint4 sgd_group(const uint4& w, const uint4& g, float lr) {
    bool nan = false;
    uint4 r;
    r.x = sgd_word(w.x, g.x, lr, nan);
    r.y = sgd_word(w.y, g.y, lr, nan);
    r.z = sgd_word(w.z, g.z, lr, nan);
    r.w = sgd_word(w.w, g.w, lr, nan);
    if (nan) {   // rare: the bf16 NaN the STE writes
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, gv[4] = {g.x, g.y, g.z, g.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = sgd_bf16_scalar(wv[i] & 0xFFFFu, gv[i] & 0xFFFFu, lr) |
                   (sgd_bf16_scalar(wv[i] >> 16, gv[i] >> 16, lr) << 16);
        r = make_uint4(o[0], o[1], o[2], o[3]);
    }
    return r;
}

// SGD on one group of bf16 latents with a float32 gradient y (the rotated
// STE's): w <- bf16(fl32(w) - fl32(lr y)), NaN -> 0x7FC0.
__device__ __forceinline__ uint4 sgd_group_f32(const uint4& w, const float (&y)[8], float lr) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float n0 = __uint_as_float(wv[i] << 16) - lr * y[2 * i];
        const float n1 = __uint_as_float(wv[i] & 0xFFFF0000u) - lr * y[2 * i + 1];
        const uint32_t u0 = __float_as_uint(n0), u1 = __float_as_uint(n1);
        const uint32_t b0 = n0 != n0 ? 0x7FC0u : (u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16;
        const uint32_t b1 = n1 != n1 ? 0x7FC0u : (u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16;
        o[i] = b0 | (b1 << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// SGD: 0 none, 1 identity STE with SGD, 2 the gradient taken back through the
// rotation, then SGD (latents updated in place before they are projected).
template <typename WT, int HB, bool FAST, bool RESTORE, int SGD = 0>
__global__ __launch_bounds__(kBlock, 6) void project_kernel(ProjectArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wv = tid >> 6;
    const uint32_t smask_words = HB > 0 ? a.cols / 2u : 0u;
    uint32_t* s_smask = s_dyn;
    float* s_wide = reinterpret_cast<float*>(s_dyn + smask_words);
    if constexpr (HB > 0) {
        load_sign_masks(s_smask, a.signs, a.cols, tid);
        __syncthreads();
    }
    const LaneFwht lf = lane_fwht<(HB > 128 ? 128 : HB)>(lane);
    const uint32_t lane_off = (lane & ~15u) + lf.logical;
    const uint32_t lpos = wv * kWave + lane_off;
    const uint32_t glast = a.groups - 1u;

    // escape counts per batch item, held back per wave while its items stay in
    // one batch item (wave-uniform, so scalar registers)
    uint32_t pend_b = 0u, pend_n = 0u;
    // Rows of at least 64 groups: a tile touches at most 65 rows, whose
    // coefficients fl32(kappa * fl32(1/s)) the block computes once per tile
    // into LDS (NaN marks a bad scale), instead of a division per group.  Not
    // in the restore and rotated-gradient forms: their register pressure made
    // them slower with it (scalar and vector spills).
    constexpr bool kRowTab = !RESTORE && SGD != 2;
    __shared__ float s_coef[kRowTab ? kTileGroups / 64u + 2u : 1u];
    const bool row_tab = kRowTab && a.gpr >= 64u;   // kernel-uniform
    for (uint32_t tile = blockIdx.x; tile < a.num_tiles; tile += gridDim.x) {
        const uint32_t tbase = tile * kTileGroups + lpos;
        uint32_t row0 = 0;
        if (row_tab) {
            row0 = fdiv(tile * kTileGroups, a.gpr_div);
            const uint32_t nrows = fdiv(min(tile * kTileGroups + (kTileGroups - 1u), glast), a.gpr_div) - row0 + 1u;
            __syncthreads();   // the previous tile's reads are done
            if (tid < nrows) {
                bool bad_r;
                const float c = row_coef(a.scale[row0 + tid], a.kappa, bad_r);
                s_coef[tid] = bad_r ? __uint_as_float(0x7FC00000u) : c;
            }
            __syncthreads();
        }
        uint32_t g1 = tbase, g2 = tbase + kBlock;
        uint32_t r1 = fdiv(min(g1, glast), a.gpr_div), r2 = fdiv(min(g2, glast), a.gpr_div);
        Raw w1 = load_raw<WT>(a.w, min(g1, glast)), w2 = load_raw<WT>(a.w, min(g2, glast));
        uint4 d1 = make_uint4(0u, 0u, 0u, 0u), d2 = d1;   // SGD: the gradient, loaded with the latents
        if constexpr (SGD) {
            d1 = load_raw<uint16_t>(a.grad, min(g1, glast)).p;
            d2 = load_raw<uint16_t>(a.grad, min(g2, glast)).p;
        }
        float s1 = a.scale[r1], s2 = a.scale[r2];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const uint32_t g = g1;
            const bool live = g < a.groups;
            const uint32_t gl = min(g, glast);
            const uint32_t row = r1;
            Raw raw = w1;
            const uint4 dg = d1;
            const float s = s1;
            g1 = g2; r1 = r2; w1 = w2; s1 = s2; d1 = d2;
            if (j + 2 < kItems) {
                g2 = g + 2u * kBlock;
                const uint32_t gn = min(g2, glast);
                r2 = fdiv(gn, a.gpr_div);
                w2 = load_raw<WT>(a.w, gn);
                if constexpr (SGD) d2 = load_raw<uint16_t>(a.grad, gn).p;
                s2 = a.scale[r2];
            }
            if constexpr (SGD == 1) {
                raw.p = sgd_group(raw.p, dg, a.lr);
                if (live) *reinterpret_cast<uint4*>(const_cast<uint16_t*>(static_cast<const uint16_t*>(a.w)) + uint64_t(g) * 8) = raw.p;
            } else if constexpr (SGD == 2 && HB > 0) {
                // dL/dw = R^T dL/dq = sigma * fl32(kappa_b H_b g) (as e8q_ste_backward_hadamard), then SGD
                Raw graw;
                graw.p = dg;
                graw.q = make_uint4(0u, 0u, 0u, 0u);
                float y[8];
                widen_raw<uint16_t>(graw, y);
                const uint32_t ys = fwht_group<HB>(y, lf, s_wide, lpos, tid);
                const float kk = __uint_as_float(__float_as_uint(a.kappa) ^ ys);
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = fmaf(y[i], kk, 0.0f);   // every zero becomes +0
                flip_f32(y, *reinterpret_cast<const uint4*>(s_smask + (gl - row * a.gpr) * 4u));
                raw.p = sgd_group_f32(raw.p, y, a.lr);
                if (live) *reinterpret_cast<uint4*>(const_cast<uint16_t*>(static_cast<const uint16_t*>(a.w)) + uint64_t(g) * 8) = raw.p;
            }
            float v[8];
            const uint32_t vsign = rotate_group<WT, HB>(s_smask, s_wide, raw, gl - row * a.gpr, lf, lpos, tid, v);
            if (HB > 0 && a.rotated && live) {
                // fma(v, kappa, +0) rounds like v * kappa and turns an exact -0 into +0
                const float kap = __uint_as_float(__float_as_uint(a.kappa) ^ vsign);
                float4* dst = reinterpret_cast<float4*>(a.rotated + uint64_t(g) * 8);
                dst[0] = make_float4(fmaf(v[0], kap, 0.0f), fmaf(v[1], kap, 0.0f), fmaf(v[2], kap, 0.0f),
                                     fmaf(v[3], kap, 0.0f));
                dst[1] = make_float4(fmaf(v[4], kap, 0.0f), fmaf(v[5], kap, 0.0f), fmaf(v[6], kap, 0.0f),
                                     fmaf(v[7], kap, 0.0f));
            }
            bool bad;
            float c0;
            if (row_tab) {
                c0 = s_coef[row - row0];
                bad = __builtin_isnan(c0);
            } else {
                c0 = row_coef(s, a.kappa, bad);
            }
            const float c = __uint_as_float(__float_as_uint(c0) ^ vsign);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = v[i] * c;
            uint32_t flags = 0;
            bool done = false;
            uint32_t norm = 0;
            float r[8];          // 2z for the restore (+64 on the fast path)
            float rcorr = 0.0f;
            if constexpr (FAST) {
                uint32_t t0, t1;
                bool d8;
                // s/2 and 32 s must be exact for the fma form of s * z
                const bool s_ok = !bad && s > 0x1p-100f && s < 0x1p100f;
                if (s_ok && fast_point(x, t0, t1, d8)) {
                    if (live && a.q) {
                        const float sh = 0.5f * s, sm = -32.0f * s;
                        float q[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            q[i] = fmaf(float((t0 >> (8 * i)) & 0xFFu), sh, sm);
                            q[4 + i] = fmaf(float((t1 >> (8 * i)) & 0xFFu), sh, sm);
                        }
                        if (a.q_bf16) {
                            uint4 p;
                            p.x = bf16x2_rne(q[0], q[1]);
                            p.y = bf16x2_rne(q[2], q[3]);
                            p.z = bf16x2_rne(q[4], q[5]);
                            p.w = bf16x2_rne(q[6], q[7]);
                            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.q) + uint64_t(g) * 8) = p;
                        } else {
                            float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.q) + uint64_t(g) * 8);
                            dst[0] = make_float4(q[0], q[1], q[2], q[3]);
                            dst[1] = make_float4(q[4], q[5], q[6], q[7]);
                        }
                    }
                    if (a.two_z && live)
                        *reinterpret_cast<uint2*>(a.two_z + uint64_t(g) * 8) = make_uint2(unbias_i8x4(t0), unbias_i8x4(t1));
                    if constexpr (RESTORE) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            r[i] = float((t0 >> (8 * i)) & 0xFFu);
                            r[4 + i] = float((t1 >> (8 * i)) & 0xFFu);
                        }
                        rcorr = 512.0f;
                    }
                    if (a.esc) {
                        const uint32_t qt = __builtin_amdgcn_udot4(t1, t1, __builtin_amdgcn_udot4(t0, t0, 0u, false), false);
                        const uint32_t st = __builtin_amdgcn_sad_u8(t1, 0u, __builtin_amdgcn_sad_u8(t0, 0u, 0u));
                        norm = qt - (st << 7) + 32768u;
                    }
                    done = true;
                }
            }
            if (!done) {
                int t[8];
                const uint32_t inv = exact_point(x, bad, t);
                if (live) flags |= inv;
                if (live && a.q) {
                    float q[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) q[i] = bad ? 0.0f : s * (float(t[i]) * 0.5f);
                    if (a.q_bf16) {
                        uint4 p;
                        p.x = pack_bf16x2(q[0], q[1]);
                        p.y = pack_bf16x2(q[2], q[3]);
                        p.z = pack_bf16x2(q[4], q[5]);
                        p.w = pack_bf16x2(q[6], q[7]);
                        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.q) + uint64_t(g) * 8) = p;
                    } else {
                        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.q) + uint64_t(g) * 8);
                        dst[0] = make_float4(q[0], q[1], q[2], q[3]);
                        dst[1] = make_float4(q[4], q[5], q[6], q[7]);
                    }
                }
                if (a.two_z && live) {
                    uint32_t f8 = 0;
                    *reinterpret_cast<uint2*>(a.two_z + uint64_t(g) * 8) = pack_i8x8(t, f8);
                    flags |= f8;
                }
                norm = norm_u32(t);
                if constexpr (RESTORE) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) r[i] = float(t[i]);
                }
            }
            if constexpr (RESTORE) {
                // inverse rotation across the block; every lane takes part
                fwht_inlane<8>(r);
                r[0] -= rcorr;
                const uint32_t rs = fwht_cross<HB>(r, lf, s_wide, lpos, tid);
                const float c2 = bad ? 0.0f : (s * a.kappa) * 0.5f;
                const float c2s = __uint_as_float(__float_as_uint(c2) ^ rs);
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = fmaf(r[i], c2s, 0.0f);   // every zero becomes +0
                if (live) {
                    const uint4 m = *reinterpret_cast<const uint4*>(s_smask + (gl - row * a.gpr) * 4u);
                    if (a.w_hat_bf16) {
                        uint4 p;
                        p.x = bf16x2_rne(y[0], y[1]) ^ m.x;
                        p.y = bf16x2_rne(y[2], y[3]) ^ m.y;
                        p.z = bf16x2_rne(y[4], y[5]) ^ m.z;
                        p.w = bf16x2_rne(y[6], y[7]) ^ m.w;
                        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.w_hat) + uint64_t(g) * 8) = p;
                    } else {
                        flip_f32(y, m);
                        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.w_hat) + uint64_t(g) * 8);
                        dst[0] = make_float4(y[0], y[1], y[2], y[3]);
                        dst[1] = make_float4(y[4], y[5], y[6], y[7]);
                    }
                }
            }
            if (a.esc) {
                const bool escaped = live && norm > uint32_t(a.core_bound);
                const uint64_t mask = __ballot(escaped);
                if (mask) {
                    const uint32_t b = live ? fdiv(g, a.gpb_div) : 0u;
                    const uint32_t b0 = __builtin_amdgcn_readfirstlane(b);
                    const bool uniform = __ballot(live && b != b0) == 0;
                    if (uniform) {
                        if (pend_n != 0u && b0 != pend_b) {
                            if (lane == 0) atomicAdd(a.esc + pend_b, (unsigned long long)pend_n);
                            pend_n = 0u;
                        }
                        pend_b = b0;
                        pend_n += uint32_t(__popcll(mask));
                    } else if (escaped) {
                        atomicAdd(a.esc + b, 1ull);
                    }
                }
            }
            flush_status(flags, a.status);
        }
    }
    if (a.esc) {
        // the block's waves pass their held counts to one thread, which adds
        // runs of equal batch items with one atomic each
        __shared__ uint32_t s_pb[kWaves], s_pn[kWaves];
        if (lane == 0) {
            s_pb[wv] = pend_b;
            s_pn[wv] = pend_n;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t rb = 0u, rn = 0u;
            for (uint32_t k = 0; k < uint32_t(kWaves); ++k) {
                if (s_pn[k] == 0u) continue;
                if (rn != 0u && s_pb[k] != rb) {
                    atomicAdd(a.esc + rb, (unsigned long long)rn);
                    rn = 0u;
                }
                rb = s_pb[k];
                rn += s_pn[k];
            }
            if (rn != 0u) atomicAdd(a.esc + rb, (unsigned long long)rn);
        }
    }
}

__global__ void zero_u64_kernel(unsigned long long* p, uint32_t n) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0ull;
}

template <typename WT, bool FAST, bool RESTORE, int SGD = 0>
static void launch_project(int hb, const ProjectArgs& a, size_t lds, hipStream_t st) {
    switch (hb) {
        case 0:  // no rotation: neither the restore nor the rotated gradient applies
            if constexpr (!RESTORE && SGD != 2)
                launch_tiles(project_kernel<WT, 0, FAST, false, SGD>, a, a.num_tiles, kBlock, lds, st);
            break;
        case 8: launch_tiles(project_kernel<WT, 8, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 16: launch_tiles(project_kernel<WT, 16, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 32: launch_tiles(project_kernel<WT, 32, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 64: launch_tiles(project_kernel<WT, 64, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 128: launch_tiles(project_kernel<WT, 128, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 256: launch_tiles(project_kernel<WT, 256, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 512: launch_tiles(project_kernel<WT, 512, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 1024: launch_tiles(project_kernel<WT, 1024, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 2048: launch_tiles(project_kernel<WT, 2048, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        case 4096: launch_tiles(project_kernel<WT, 4096, FAST, RESTORE, SGD>, a, a.num_tiles, kBlock, lds, st); break;
        default: break;
    }
}

static e8q_status_t project_impl(const void* w, e8q_dtype_t w_dtype, int64_t batch, int64_t rows,
                                 int64_t cols, const float* row_scale, const int8_t* signs,
                                 int32_t had_block, void* q_out, e8q_dtype_t q_dtype,
                                 int8_t* two_z_out, float* rotated_out, int32_t core_bound,
                                 int64_t* esc_count_out, uint32_t* status_dev, void* stream,
                                 void* w_hat_out = nullptr, e8q_dtype_t w_hat_dtype = E8Q_F32,
                                 const void* grad = nullptr, float lr = 0.0f, bool rotate_grad = false) {
    e8q_status_t st = check_shape(w, w_dtype, batch, rows, cols, row_scale, status_dev);
    if (st != E8Q_OK) return st;
    if (!q_out && !two_z_out && !esc_count_out && !rotated_out && !w_hat_out) return E8Q_ERR_INVALID;
    if (w_hat_out && (had_block < 8 || (w_hat_dtype != E8Q_F32 && w_hat_dtype != E8Q_BF16)))
        return E8Q_ERR_INVALID;
    if (q_out && q_dtype != E8Q_F32 && q_dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    if (esc_count_out && core_bound < 0) return E8Q_ERR_INVALID;
    const size_t lds = (had_block > 0 ? size_t(cols / 2) * 4 : 0) + (had_block > 128 ? size_t(8 * kBlock) * 4 : 0);
    if (lds > 60 * 1024) return E8Q_ERR_UNSUPPORTED;   // rows too wide for the LDS sign masks

    const uint32_t gpr = uint32_t(cols / 8);
    const uint64_t groups = uint64_t(batch) * uint64_t(rows) * gpr;
    ProjectArgs a;
    a.w = w;
    a.groups = uint32_t(groups);
    a.gpr = gpr;
    a.gpr_div = make_fastdiv(gpr);
    a.gpb_div = make_fastdiv(uint32_t(uint64_t(rows) * gpr));
    a.scale = row_scale;
    a.signs = signs;
    a.cols = uint32_t(cols);
    a.kappa = kappa_for(had_block);
    a.q = q_out;
    a.q_bf16 = q_dtype == E8Q_BF16;
    a.two_z = two_z_out;
    a.rotated = rotated_out;
    a.core_bound = core_bound;
    a.esc = reinterpret_cast<unsigned long long*>(esc_count_out);
    a.status = status_dev;
    a.num_tiles = uint32_t((groups + kTileGroups - 1) / kTileGroups);
    a.w_hat = w_hat_out;
    a.w_hat_bf16 = w_hat_dtype == E8Q_BF16;
    a.grad = grad;
    a.lr = lr;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (esc_count_out) {
        launch(zero_u64_kernel, dim3(unsigned((batch + 255) / 256)), dim3(256), 0, s,
                           a.esc, uint32_t(batch));
    }
    if (grad && rotate_grad) {
        launch_project<uint16_t, true, false, 2>(had_block, a, lds, s);
    } else if (grad && w_hat_out) {
        launch_project<uint16_t, true, true, 1>(had_block, a, lds, s);
    } else if (grad) {
        launch_project<uint16_t, true, false, 1>(had_block, a, lds, s);
    } else if (w_hat_out) {
        if (w_dtype == E8Q_BF16)
            launch_project<uint16_t, true, true>(had_block, a, lds, s);
        else
            launch_project<float, false, true>(had_block, a, lds, s);
    } else if (w_dtype == E8Q_BF16) {
        launch_project<uint16_t, true, false>(had_block, a, lds, s);
    } else {
        launch_project<float, false, false>(had_block, a, lds, s);
    }
    return launch_status();
}

}  // namespace e8q

extern "C" e8q_status_t e8q_project(const void* w, e8q_dtype_t w_dtype, int64_t batch, int64_t rows,
                                    int64_t cols, const float* row_scale, void* q_out,
                                    e8q_dtype_t q_dtype, int8_t* two_z_out, int32_t core_bound,
                                    int64_t* esc_count_out, uint32_t* status_dev, void* stream) {
    return e8q::project_impl(w, w_dtype, batch, rows, cols, row_scale, nullptr, 0, q_out, q_dtype,
                             two_z_out, nullptr, core_bound, esc_count_out, status_dev, stream);
}

extern "C" e8q_status_t e8q_project_hadamard(const void* w, e8q_dtype_t w_dtype, int64_t batch,
                                             int64_t rows, int64_t cols, const float* row_scale,
                                             const int8_t* signs, int32_t had_block, void* q_out,
                                             e8q_dtype_t q_dtype, int8_t* two_z_out,
                                             float* rotated_out, int32_t core_bound,
                                             int64_t* esc_count_out, uint32_t* status_dev,
                                             void* stream) {
    e8q_status_t st = e8q::check_block(signs, had_block, cols);
    if (st != E8Q_OK) return st;
    return e8q::project_impl(w, w_dtype, batch, rows, cols, row_scale, signs, had_block, q_out,
                             q_dtype, two_z_out, rotated_out, core_bound, esc_count_out, status_dev,
                             stream);
}

extern "C" e8q_status_t e8q_project_hadamard_restore(const void* w, e8q_dtype_t w_dtype, int64_t batch,
                                                     int64_t rows, int64_t cols, const float* row_scale,
                                                     const int8_t* signs, int32_t had_block, void* w_hat_out,
                                                     e8q_dtype_t w_hat_dtype, int8_t* two_z_out,
                                                     int32_t core_bound, int64_t* esc_count_out,
                                                     uint32_t* status_dev, void* stream) {
    e8q_status_t st = e8q::check_block(signs, had_block, cols);
    if (st != E8Q_OK) return st;
    if (!w_hat_out) return E8Q_ERR_INVALID;
    return e8q::project_impl(w, w_dtype, batch, rows, cols, row_scale, signs, had_block, nullptr, E8Q_F32,
                             two_z_out, nullptr, core_bound, esc_count_out, status_dev, stream, w_hat_out,
                             w_hat_dtype);
}

extern "C" e8q_status_t e8q_sgd_project_hadamard(void* w_latent, const void* grad, float lr, int64_t batch,
                                                 int64_t rows, int64_t cols, const float* row_scale,
                                                 const int8_t* signs, int32_t had_block, void* q_out,
                                                 e8q_dtype_t q_dtype, int8_t* two_z_out, int32_t core_bound,
                                                 int64_t* esc_count_out, uint32_t* status_dev, void* stream) {
    if (!w_latent || !grad) return E8Q_ERR_INVALID;
    if (signs) {
        const e8q_status_t st = e8q::check_block(signs, had_block, cols);
        if (st != E8Q_OK) return st;
    }
    return e8q::project_impl(w_latent, E8Q_BF16, batch, rows, cols, row_scale, signs, signs ? had_block : 0, q_out,
                             q_dtype, two_z_out, nullptr, core_bound, esc_count_out, status_dev, stream, nullptr,
                             E8Q_F32, grad, lr);
}

extern "C" e8q_status_t e8q_sgd_project_hadamard_restore(void* w_latent, const void* grad, float lr, int64_t batch,
                                                         int64_t rows, int64_t cols, const float* row_scale,
                                                         const int8_t* signs, int32_t had_block, void* w_hat_out,
                                                         e8q_dtype_t w_hat_dtype, int8_t* two_z_out,
                                                         int32_t core_bound, int64_t* esc_count_out,
                                                         uint32_t* status_dev, void* stream) {
    if (!w_latent || !grad || !w_hat_out) return E8Q_ERR_INVALID;
    const e8q_status_t st = e8q::check_block(signs, had_block, cols);
    if (st != E8Q_OK) return st;
    return e8q::project_impl(w_latent, E8Q_BF16, batch, rows, cols, row_scale, signs, had_block, nullptr, E8Q_F32,
                             two_z_out, nullptr, core_bound, esc_count_out, status_dev, stream, w_hat_out,
                             w_hat_dtype, grad, lr);
}

extern "C" e8q_status_t e8q_sgd_rotated_project_hadamard(void* w_latent, const void* grad_q, float lr, int64_t batch,
                                                         int64_t rows, int64_t cols, const float* row_scale,
                                                         const int8_t* signs, int32_t had_block, void* q_out,
                                                         e8q_dtype_t q_dtype, int8_t* two_z_out, int32_t core_bound,
                                                         int64_t* esc_count_out, uint32_t* status_dev,
                                                         void* stream) {
    if (!w_latent || !grad_q) return E8Q_ERR_INVALID;
    const e8q_status_t st = e8q::check_block(signs, had_block, cols);
    if (st != E8Q_OK) return st;
    return e8q::project_impl(w_latent, E8Q_BF16, batch, rows, cols, row_scale, signs, had_block, q_out, q_dtype,
                             two_z_out, nullptr, core_bound, esc_count_out, status_dev, stream, nullptr, E8Q_F32,
                             grad_q, lr, true);
}
