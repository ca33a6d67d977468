// e8q_project / e8q_project_hadamard: the QAT forward projection.
//
// E8-QAT maps every group of eight normalized weights to its nearest E8 point
// by arithmetic in every training forward pass (abstract; Figure 1(c) and
// Figure 2(b) captions), after a Hadamard transform and with reconstruction
// scales that the overview figure leaves out (Figure 2 caption).  This kernel
// is a streaming map: one 16-byte load and one 16-byte store per lane per
// group (bf16), Walsh-Hadamard butterflies in registers and across the lanes
// of one 16-lane DPP row, and the round-and-fix-parity decoder per lane.
#include "e8q_device.hpp"
#include "e8q_host.hpp"

namespace e8q {

struct ProjectArgs {
    const void* w;
    uint32_t groups;          // batch*rows*cols/8
    uint32_t gpr;             // groups per row
    FastDiv gpr_div;
    FastDiv gpb_div;          // groups per batch item
    const float* scale;
    const int8_t* signs;
    float kappa;
    void* q;
    int q_bf16;
    int8_t* two_z;
    float* rotated;
    int core_bound;
    unsigned long long* esc;
    uint32_t* status;
};

template <typename WT, int HB>
__global__ __launch_bounds__(256) void project_kernel(ProjectArgs a) {
    const uint32_t lane = __lane_id();
    const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const uint32_t nwaves = gridDim.x * blockDim.x / kWave;
    const LaneFwht lf = lane_fwht<HB>(lane);
    const uint32_t lane_off = (lane & ~15u) + lf.logical;
    for (uint64_t base = uint64_t(wave) * kWave; base < a.groups; base += uint64_t(nwaves) * kWave) {
        const uint32_t g = uint32_t(base) + lane_off;
        const bool live = g < a.groups;
        float v[8];
        if (live) {
            load_group(reinterpret_cast<const WT*>(a.w), g, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        }
        const uint32_t row = live ? fdiv(g, a.gpr_div) : 0u;
        const uint32_t col0 = (g - row * a.gpr) * 8u;
        float kap = a.kappa;
        if constexpr (HB > 0) {
            if (live) apply_signs(a.signs, col0, v);
            fwht_inlane<HB>(v);
            fwht_xlane<HB>(v, lf.eps);
            // the lane holds the transform times (-1)^popcount(L): fold it in
            kap = __uint_as_float(__float_as_uint(kap) ^ lf.sign);
            if (a.rotated && live) {
                float4* dst = reinterpret_cast<float4*>(a.rotated + uint64_t(g) * 8);
                // fma(v, kap, +0) rounds like v * kap and turns an exact -0 into +0
                dst[0] = make_float4(fmaf(v[0], kap, 0.0f), fmaf(v[1], kap, 0.0f), fmaf(v[2], kap, 0.0f),
                                     fmaf(v[3], kap, 0.0f));
                dst[1] = make_float4(fmaf(v[4], kap, 0.0f), fmaf(v[5], kap, 0.0f), fmaf(v[6], kap, 0.0f),
                                     fmaf(v[7], kap, 0.0f));
            }
        }
        const float s = a.scale[row];
        bool bad;
        const float c0 = row_coef(s, a.kappa, bad);
        const float c = __uint_as_float(__float_as_uint(c0) ^ (HB > 0 ? lf.sign : 0u));
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = v[i] * c;
        uint32_t flags = 0;
        int t[8];
        if (bad) {
            flags = live ? uint32_t(E8Q_STATUS_BAD_SCALE) : 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = 0;
        } else {
            const uint32_t inv = group_invalid_bits(x);
            if (inv) {
                flags = live ? inv : 0u;
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = 0;
            } else {
                nearest_e8(x, t);
            }
        }
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
        if (a.two_z) {
            uint32_t f8 = 0;
            const uint2 p = pack_i8x8(t, f8);
            if (live) {
                *reinterpret_cast<uint2*>(a.two_z + uint64_t(g) * 8) = p;
                flags |= f8;
            }
        }
        if (a.esc) {
            uint32_t norm = 0;   // <= 8 * 16386^2 < 2^32
#pragma unroll
            for (int i = 0; i < 8; ++i) norm += uint32_t(t[i] * t[i]);
            const bool escaped = live && norm > uint32_t(a.core_bound);
            const uint64_t mask = __ballot(escaped);
            if (mask) {
                const uint32_t b = live ? fdiv(g, a.gpb_div) : 0u;
                const uint32_t b0 = __shfl(b, 0, 64);
                const bool uniform = __ballot(live && b != b0) == 0;
                if (uniform) {
                    if (lane == 0) atomicAdd(a.esc + b0, (unsigned long long)__popcll(mask));
                } else if (escaped) {
                    atomicAdd(a.esc + b, 1ull);
                }
            }
        }
        flush_status(flags, a.status);
    }
}

__global__ void zero_u64_kernel(unsigned long long* p, uint32_t n) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0ull;
}

template <typename WT>
static void launch_project(int hb, const ProjectArgs& a, unsigned grid, hipStream_t st) {
    switch (hb) {
        case 0: hipLaunchKernelGGL((project_kernel<WT, 0>), dim3(grid), dim3(256), 0, st, a); break;
        case 8: hipLaunchKernelGGL((project_kernel<WT, 8>), dim3(grid), dim3(256), 0, st, a); break;
        case 16: hipLaunchKernelGGL((project_kernel<WT, 16>), dim3(grid), dim3(256), 0, st, a); break;
        case 32: hipLaunchKernelGGL((project_kernel<WT, 32>), dim3(grid), dim3(256), 0, st, a); break;
        case 64: hipLaunchKernelGGL((project_kernel<WT, 64>), dim3(grid), dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL((project_kernel<WT, 128>), dim3(grid), dim3(256), 0, st, a); break;
        default: break;
    }
}

static e8q_status_t project_impl(const void* w, e8q_dtype_t w_dtype, int64_t batch, int64_t rows,
                                 int64_t cols, const float* row_scale, const int8_t* signs,
                                 int32_t had_block, void* q_out, e8q_dtype_t q_dtype,
                                 int8_t* two_z_out, float* rotated_out, int32_t core_bound,
                                 int64_t* esc_count_out, uint32_t* status_dev, void* stream) {
    e8q_status_t st = check_shape(w, w_dtype, batch, rows, cols, row_scale, status_dev);
    if (st != E8Q_OK) return st;
    if (!q_out && !two_z_out && !esc_count_out && !rotated_out) return E8Q_ERR_INVALID;
    if (q_out && q_dtype != E8Q_F32 && q_dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    if (esc_count_out && core_bound < 0) return E8Q_ERR_INVALID;
    if (had_block > 128) return E8Q_ERR_UNSUPPORTED;   // wider blocks: not in this build

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
    a.kappa = kappa_for(had_block);
    a.q = q_out;
    a.q_bf16 = q_dtype == E8Q_BF16;
    a.two_z = two_z_out;
    a.rotated = rotated_out;
    a.core_bound = core_bound;
    a.esc = reinterpret_cast<unsigned long long*>(esc_count_out);
    a.status = status_dev;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (esc_count_out) {
        hipLaunchKernelGGL(zero_u64_kernel, dim3(unsigned((batch + 255) / 256)), dim3(256), 0, s,
                           a.esc, uint32_t(batch));
    }
    const unsigned grid = grid_for(groups, 256, 8);
    if (w_dtype == E8Q_BF16)
        launch_project<uint16_t>(had_block, a, grid, s);
    else
        launch_project<float>(had_block, a, grid, s);
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
