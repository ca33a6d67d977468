// Forward rotation of whole rows without projection: xt = kappa * H_b (sigma * x)
// per block (kappa = 1 gives the un-normalized transform), on the projection's
// tile layout and lanes.  Used to rotate GEMV activations once per vector and
// to precompute the transform of the weights for the PTQ scale search.
#pragma once

#include "e8q_host.hpp"
#include "e8q_point.hpp"

namespace e8q {

struct RotArgs {
    const void* x;
    float* xt;
    const int8_t* signs;
    float kappa;
    uint32_t cols;
    uint32_t groups;
    uint32_t gpr;
    FastDiv gpr_div;
    uint32_t num_tiles;
};

template <typename WT, int HB>
__global__ __launch_bounds__(kBlock) void rotate_act_kernel(RotArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wv = tid >> 6;
    uint32_t* s_smask = s_dyn;
    float* s_wide = reinterpret_cast<float*>(s_dyn + (HB > 0 ? a.cols / 2u : 0u));
    if constexpr (HB > 0) {
        load_sign_masks(s_smask, a.signs, a.cols, tid);
        __syncthreads();
    }
    const LaneFwht lf = lane_fwht<(HB > 128 ? 128 : HB)>(lane);
    const uint32_t lpos = wv * kWave + (lane & ~15u) + lf.logical;
    const uint32_t glast = a.groups - 1u;
    for (uint32_t tile = blockIdx.x; tile < a.num_tiles; tile += gridDim.x) {
#pragma unroll 1
        for (int j = 0; j < kItems; ++j) {
            const uint32_t g = tile * kTileGroups + uint32_t(j) * kBlock + lpos;
            const uint32_t gl = min(g, glast);
            const Raw raw = load_raw<WT>(a.x, gl);
            float v[8];
            const uint32_t vs = rotate_group<WT, HB>(s_smask, s_wide, raw, gl - fdiv(gl, a.gpr_div) * a.gpr, lf, lpos,
                                                     tid, v);
            const float k = __uint_as_float(__float_as_uint(a.kappa) ^ vs);
            if (g < a.groups) {
                float4* dst = reinterpret_cast<float4*>(a.xt + uint64_t(g) * 8);
                dst[0] = make_float4(v[0] * k, v[1] * k, v[2] * k, v[3] * k);
                dst[1] = make_float4(v[4] * k, v[5] * k, v[6] * k, v[7] * k);
            }
        }
    }
}

template <typename WT>
inline void launch_rotate(int hb, const RotArgs& a, size_t lds, hipStream_t st) {
    switch (hb) {
        case 0: launch_tiles(rotate_act_kernel<WT, 0>, a, a.num_tiles, kBlock, lds, st); break;
        case 8: launch_tiles(rotate_act_kernel<WT, 8>, a, a.num_tiles, kBlock, lds, st); break;
        case 16: launch_tiles(rotate_act_kernel<WT, 16>, a, a.num_tiles, kBlock, lds, st); break;
        case 32: launch_tiles(rotate_act_kernel<WT, 32>, a, a.num_tiles, kBlock, lds, st); break;
        case 64: launch_tiles(rotate_act_kernel<WT, 64>, a, a.num_tiles, kBlock, lds, st); break;
        case 128: launch_tiles(rotate_act_kernel<WT, 128>, a, a.num_tiles, kBlock, lds, st); break;
        case 256: launch_tiles(rotate_act_kernel<WT, 256>, a, a.num_tiles, kBlock, lds, st); break;
        case 512: launch_tiles(rotate_act_kernel<WT, 512>, a, a.num_tiles, kBlock, lds, st); break;
        case 1024: launch_tiles(rotate_act_kernel<WT, 1024>, a, a.num_tiles, kBlock, lds, st); break;
        case 2048: launch_tiles(rotate_act_kernel<WT, 2048>, a, a.num_tiles, kBlock, lds, st); break;
        case 4096: launch_tiles(rotate_act_kernel<WT, 4096>, a, a.num_tiles, kBlock, lds, st); break;
        default: break;
    }
}

}  // namespace e8q
