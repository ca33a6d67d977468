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
    uint4* xb;        // optional: x~ split into three bfloat16 parts, [rows of x, 3, gpr] x 8 bf16
    const int8_t* signs;
    float kappa;
    uint32_t cols;
    uint32_t groups;
    uint32_t gpr;
    FastDiv gpr_div;
    uint32_t num_tiles;
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
}

// x = hi + mid + lo, each the bfloat16 (round to nearest even) of what the
// earlier parts leave (both differences exact; |x - hi - mid - lo| <= 2^-24 |x|).
__device__ __forceinline__ void split3_bf16(const float (&x)[8], uint4& h, uint4& m, uint4& l) {
    uint32_t hh[8], mm[8], ll[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t hb = bf16_rne_bits(x[i]);
        const float d = x[i] - __uint_as_float(hb);
        const uint32_t mb = bf16_rne_bits(d);
        const float e = d - __uint_as_float(mb);
        hh[i] = hb >> 16;
        mm[i] = mb >> 16;
        ll[i] = bf16_rne_bits(e) >> 16;
    }
    h = make_uint4(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16), hh[4] | (hh[5] << 16), hh[6] | (hh[7] << 16));
    m = make_uint4(mm[0] | (mm[1] << 16), mm[2] | (mm[3] << 16), mm[4] | (mm[5] << 16), mm[6] | (mm[7] << 16));
    l = make_uint4(ll[0] | (ll[1] << 16), ll[2] | (ll[3] << 16), ll[4] | (ll[5] << 16), ll[6] | (ll[7] << 16));
}

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
    // one item (kBlock groups) of a tile per step, so that short inputs (an
    // activation vector per batch item) still spread over many blocks
    for (uint32_t ti = blockIdx.x; ti < a.num_tiles * uint32_t(kItems); ti += gridDim.x) {
        {
            const uint32_t tile = ti / uint32_t(kItems), j = ti - tile * uint32_t(kItems);
            const uint32_t g = tile * kTileGroups + j * kBlock + lpos;
            const uint32_t gl = min(g, glast);
            const Raw raw = load_raw<WT>(a.x, gl);
            float v[8];
            const uint32_t row = fdiv(gl, a.gpr_div);
            const uint32_t gi = gl - row * a.gpr;
            const uint32_t vs = rotate_group<WT, HB>(s_smask, s_wide, raw, gi, lf, lpos, tid, v);
            const float k = __uint_as_float(__float_as_uint(a.kappa) ^ vs);
            if (g < a.groups) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = v[i] * k;
                float4* dst = reinterpret_cast<float4*>(a.xt + uint64_t(g) * 8);
                dst[0] = make_float4(y[0], y[1], y[2], y[3]);
                dst[1] = make_float4(y[4], y[5], y[6], y[7]);
                if (a.xb) {
                    uint4 h, m, l;
                    split3_bf16(y, h, m, l);
                    uint4* pb = a.xb + uint64_t(row) * 3u * a.gpr + gi;
                    pb[0] = h;
                    pb[a.gpr] = m;
                    pb[2u * a.gpr] = l;
                }
            }
        }
    }
}

template <typename K>
inline void launch_tiles_items(K kernel, const RotArgs& a, uint64_t tiles, unsigned block, size_t lds, hipStream_t st) {
    launch_tiles(kernel, a, tiles * uint64_t(kItems), block, lds, st);
}

template <typename WT>
inline void launch_rotate(int hb, const RotArgs& a, size_t lds, hipStream_t st) {
    switch (hb) {
        case 0: launch_tiles_items(rotate_act_kernel<WT, 0>, a, a.num_tiles, kBlock, lds, st); break;
        case 8: launch_tiles_items(rotate_act_kernel<WT, 8>, a, a.num_tiles, kBlock, lds, st); break;
        case 16: launch_tiles_items(rotate_act_kernel<WT, 16>, a, a.num_tiles, kBlock, lds, st); break;
        case 32: launch_tiles_items(rotate_act_kernel<WT, 32>, a, a.num_tiles, kBlock, lds, st); break;
        case 64: launch_tiles_items(rotate_act_kernel<WT, 64>, a, a.num_tiles, kBlock, lds, st); break;
        case 128: launch_tiles_items(rotate_act_kernel<WT, 128>, a, a.num_tiles, kBlock, lds, st); break;
        case 256: launch_tiles_items(rotate_act_kernel<WT, 256>, a, a.num_tiles, kBlock, lds, st); break;
        case 512: launch_tiles_items(rotate_act_kernel<WT, 512>, a, a.num_tiles, kBlock, lds, st); break;
        case 1024: launch_tiles_items(rotate_act_kernel<WT, 1024>, a, a.num_tiles, kBlock, lds, st); break;
        case 2048: launch_tiles_items(rotate_act_kernel<WT, 2048>, a, a.num_tiles, kBlock, lds, st); break;
        case 4096: launch_tiles_items(rotate_act_kernel<WT, 4096>, a, a.num_tiles, kBlock, lds, st); break;
        default: break;
    }
}

}  // namespace e8q
