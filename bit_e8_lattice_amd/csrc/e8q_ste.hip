// e8q_ste_backward: identity straight-through estimator, optionally fused with
// the SGD step on the latent weights.
//
// E8-QAT trains through the projection with an identity STE (Figure 2(b)
// caption), so dL/dw = dL/dq bit for bit; latents are BF16 (Table 4).  The
// fused update reads g and w once and writes w once: 16-byte vector accesses,
// a pure HBM stream.
//
// e8q_ste_backward_hadamard is the same estimator for a projection whose
// output stays in the rotated basis: dL/dw = R^T dL/dq with R the forward
// rotation (sign flip, blockwise Walsh-Hadamard transform, kappa_b), i.e.
// sigma * fl32(kappa_b * H_b g) -- the transform on the forward's lanes, then
// the sign flip.  Each thread owns whole groups, as in the projection.
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"

namespace e8q {

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if (f != f) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t sgd_bf16x2(uint32_t w2, uint32_t g2, float lr) {
    const float w0 = __uint_as_float(w2 << 16), w1 = __uint_as_float(w2 & 0xFFFF0000u);
    const float g0 = __uint_as_float(g2 << 16), g1 = __uint_as_float(g2 & 0xFFFF0000u);
    const float n0 = w0 - lr * g0;
    const float n1 = w1 - lr * g1;
    return f32_to_bf16_rne(n0) | (f32_to_bf16_rne(n1) << 16);
}

// n16 = number of 16-byte chunks; tail elements handled by the scalar kernel.
__global__ __launch_bounds__(256) void ste_bf16_kernel(const uint4* __restrict__ g, uint4* gw,
                                                       uint4* wl, float lr, uint64_t n16) {
    for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += uint64_t(gridDim.x) * blockDim.x) {
        const uint4 gv = g[i];
        if (gw) gw[i] = gv;
        if (wl) {
            uint4 wv = wl[i];
            wv.x = sgd_bf16x2(wv.x, gv.x, lr);
            wv.y = sgd_bf16x2(wv.y, gv.y, lr);
            wv.z = sgd_bf16x2(wv.z, gv.z, lr);
            wv.w = sgd_bf16x2(wv.w, gv.w, lr);
            wl[i] = wv;
        }
    }
}

__global__ __launch_bounds__(256) void ste_f32_kernel(const float4* __restrict__ g, float4* gw,
                                                      float4* wl, float lr, uint64_t n16) {
    for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += uint64_t(gridDim.x) * blockDim.x) {
        const float4 gv = g[i];
        if (gw) gw[i] = gv;
        if (wl) {
            float4 wv = wl[i];
            wv.x = wv.x - lr * gv.x;
            wv.y = wv.y - lr * gv.y;
            wv.z = wv.z - lr * gv.z;
            wv.w = wv.w - lr * gv.w;
            wl[i] = wv;
        }
    }
}

// Elements that do not fill a 16-byte chunk (and unaligned pointers).
__global__ void ste_tail_kernel(const void* g, void* gw, void* wl, float lr, int is_bf16,
                                uint64_t lo, uint64_t n) {
    for (uint64_t i = lo + uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += uint64_t(gridDim.x) * blockDim.x) {
        if (is_bf16) {
            const uint16_t gv = static_cast<const uint16_t*>(g)[i];
            if (gw) static_cast<uint16_t*>(gw)[i] = gv;
            if (wl) {
                uint16_t* w = static_cast<uint16_t*>(wl);
                const float nv = __uint_as_float(uint32_t(w[i]) << 16) - lr * __uint_as_float(uint32_t(gv) << 16);
                w[i] = uint16_t(f32_to_bf16_rne(nv));
            }
        } else {
            const float gv = static_cast<const float*>(g)[i];
            if (gw) static_cast<float*>(gw)[i] = gv;
            if (wl) static_cast<float*>(wl)[i] = static_cast<float*>(wl)[i] - lr * gv;
        }
    }
}

struct SteHadArgs {
    const void* g;
    void* gw;
    void* wl;
    float lr;
    float kappa;
    const int8_t* signs;
    uint32_t cols;
    uint32_t groups;
    uint32_t gpr;
    FastDiv gpr_div;
    uint32_t num_tiles;
};

template <typename WT, int HB>
__global__ __launch_bounds__(kBlock) void ste_hadamard_kernel(SteHadArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wv = tid >> 6;
    uint32_t* s_smask = s_dyn;
    float* s_wide = reinterpret_cast<float*>(s_dyn + a.cols / 2u);
    load_sign_masks(s_smask, a.signs, a.cols, tid);
    __syncthreads();
    const LaneFwht lf = lane_fwht<(HB > 128 ? 128 : HB)>(lane);
    const uint32_t lpos = wv * kWave + (lane & ~15u) + lf.logical;
    const uint32_t glast = a.groups - 1u;

    for (uint32_t tile = blockIdx.x; tile < a.num_tiles; tile += gridDim.x) {
        const uint32_t tbase = tile * kTileGroups + lpos;
        uint32_t g1 = tbase, g2 = tbase + kBlock;
        Raw r1 = load_raw<WT>(a.g, min(g1, glast)), r2 = load_raw<WT>(a.g, min(g2, glast));
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const uint32_t g = g1;
            const bool live = g < a.groups;
            const uint32_t gl = min(g, glast);
            const Raw raw = r1;
            g1 = g2; r1 = r2;
            if (j + 2 < kItems) {
                g2 = g + 2u * kBlock;
                r2 = load_raw<WT>(a.g, min(g2, glast));
            }
            float v[8];
            widen_raw<WT>(raw, v);
            const uint32_t vs = fwht_group<HB>(v, lf, s_wide, lpos, tid);
            const float k = __uint_as_float(__float_as_uint(a.kappa) ^ vs);
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = fmaf(v[i], k, 0.0f);   // every zero becomes +0
            const uint32_t col_group = gl - fdiv(gl, a.gpr_div) * a.gpr;
            flip_f32(y, *reinterpret_cast<const uint4*>(s_smask + col_group * 4u));
            if (!live) continue;
            if constexpr (sizeof(WT) == 2) {
                if (a.gw) {
                    uint4 p;
                    p.x = f32_to_bf16_rne(y[0]) | (f32_to_bf16_rne(y[1]) << 16);
                    p.y = f32_to_bf16_rne(y[2]) | (f32_to_bf16_rne(y[3]) << 16);
                    p.z = f32_to_bf16_rne(y[4]) | (f32_to_bf16_rne(y[5]) << 16);
                    p.w = f32_to_bf16_rne(y[6]) | (f32_to_bf16_rne(y[7]) << 16);
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.gw) + uint64_t(g) * 8) = p;
                }
                if (a.wl) {
                    uint4* wp = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.wl) + uint64_t(g) * 8);
                    const uint4 wr = *wp;
                    float n[8];
                    n[0] = __uint_as_float(wr.x << 16) - a.lr * y[0];
                    n[1] = __uint_as_float(wr.x & 0xFFFF0000u) - a.lr * y[1];
                    n[2] = __uint_as_float(wr.y << 16) - a.lr * y[2];
                    n[3] = __uint_as_float(wr.y & 0xFFFF0000u) - a.lr * y[3];
                    n[4] = __uint_as_float(wr.z << 16) - a.lr * y[4];
                    n[5] = __uint_as_float(wr.z & 0xFFFF0000u) - a.lr * y[5];
                    n[6] = __uint_as_float(wr.w << 16) - a.lr * y[6];
                    n[7] = __uint_as_float(wr.w & 0xFFFF0000u) - a.lr * y[7];
                    uint4 p;
                    p.x = f32_to_bf16_rne(n[0]) | (f32_to_bf16_rne(n[1]) << 16);
                    p.y = f32_to_bf16_rne(n[2]) | (f32_to_bf16_rne(n[3]) << 16);
                    p.z = f32_to_bf16_rne(n[4]) | (f32_to_bf16_rne(n[5]) << 16);
                    p.w = f32_to_bf16_rne(n[6]) | (f32_to_bf16_rne(n[7]) << 16);
                    *wp = p;
                }
            } else {
                if (a.gw) {
                    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.gw) + uint64_t(g) * 8);
                    dst[0] = make_float4(y[0], y[1], y[2], y[3]);
                    dst[1] = make_float4(y[4], y[5], y[6], y[7]);
                }
                if (a.wl) {
                    float4* wp = reinterpret_cast<float4*>(static_cast<float*>(a.wl) + uint64_t(g) * 8);
                    float4 w0 = wp[0], w1 = wp[1];
                    w0.x = w0.x - a.lr * y[0]; w0.y = w0.y - a.lr * y[1];
                    w0.z = w0.z - a.lr * y[2]; w0.w = w0.w - a.lr * y[3];
                    w1.x = w1.x - a.lr * y[4]; w1.y = w1.y - a.lr * y[5];
                    w1.z = w1.z - a.lr * y[6]; w1.w = w1.w - a.lr * y[7];
                    wp[0] = w0;
                    wp[1] = w1;
                }
            }
        }
    }
}

template <typename WT>
static void launch_ste_hadamard(int hb, const SteHadArgs& a, size_t lds, hipStream_t st) {
    switch (hb) {
        case 8: launch_tiles(ste_hadamard_kernel<WT, 8>, a, a.num_tiles, kBlock, lds, st); break;
        case 16: launch_tiles(ste_hadamard_kernel<WT, 16>, a, a.num_tiles, kBlock, lds, st); break;
        case 32: launch_tiles(ste_hadamard_kernel<WT, 32>, a, a.num_tiles, kBlock, lds, st); break;
        case 64: launch_tiles(ste_hadamard_kernel<WT, 64>, a, a.num_tiles, kBlock, lds, st); break;
        case 128: launch_tiles(ste_hadamard_kernel<WT, 128>, a, a.num_tiles, kBlock, lds, st); break;
        case 256: launch_tiles(ste_hadamard_kernel<WT, 256>, a, a.num_tiles, kBlock, lds, st); break;
        case 512: launch_tiles(ste_hadamard_kernel<WT, 512>, a, a.num_tiles, kBlock, lds, st); break;
        case 1024: launch_tiles(ste_hadamard_kernel<WT, 1024>, a, a.num_tiles, kBlock, lds, st); break;
        case 2048: launch_tiles(ste_hadamard_kernel<WT, 2048>, a, a.num_tiles, kBlock, lds, st); break;
        case 4096: launch_tiles(ste_hadamard_kernel<WT, 4096>, a, a.num_tiles, kBlock, lds, st); break;
        default: break;
    }
}

}  // namespace e8q

extern "C" e8q_status_t e8q_ste_backward_hadamard(const void* grad_q, e8q_dtype_t dtype, int64_t rows,
                                                  int64_t cols, const int8_t* signs, int32_t had_block,
                                                  void* grad_w, void* w_latent, float lr, void* stream) {
    using namespace e8q;
    if (!grad_q || rows <= 0 || cols <= 0 || (!grad_w && !w_latent)) return E8Q_ERR_INVALID;
    if (dtype != E8Q_F32 && dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    if (w_latent && (w_latent == grad_q || w_latent == grad_w)) return E8Q_ERR_INVALID;
    e8q_status_t st = check_block(signs, had_block, cols);
    if (st != E8Q_OK) return st;
    const double groups = double(rows) * double(cols / 8);
    if (groups >= 4294967295.0) return E8Q_ERR_UNSUPPORTED;
    const size_t lds = size_t(cols / 2) * 4 + (had_block > 128 ? size_t(8 * kBlock) * 4 : 0);
    if (lds > 60 * 1024) return E8Q_ERR_UNSUPPORTED;
    SteHadArgs a;
    a.g = grad_q;
    a.gw = grad_w;
    a.wl = w_latent;
    a.lr = lr;
    a.kappa = kappa_for(had_block);
    a.signs = signs;
    a.cols = uint32_t(cols);
    a.groups = uint32_t(uint64_t(rows) * uint64_t(cols / 8));
    a.gpr = uint32_t(cols / 8);
    a.gpr_div = make_fastdiv(a.gpr);
    a.num_tiles = uint32_t((uint64_t(a.groups) + kTileGroups - 1) / kTileGroups);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dtype == E8Q_BF16)
        launch_ste_hadamard<uint16_t>(had_block, a, lds, s);
    else
        launch_ste_hadamard<float>(had_block, a, lds, s);
    return launch_status();
}

extern "C" e8q_status_t e8q_ste_backward(const void* grad_q, void* grad_w, void* w_latent, float lr,
                                         e8q_dtype_t dtype, int64_t n, void* stream) {
    using namespace e8q;
    if (!grad_q || n <= 0 || (!grad_w && !w_latent)) return E8Q_ERR_INVALID;
    if (dtype != E8Q_F32 && dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    const size_t esz = dtype == E8Q_BF16 ? 2 : 4;
    if (grad_w && (grad_w == grad_q || grad_w == w_latent)) return E8Q_ERR_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    uint64_t vec = 0;
    if (aligned(grad_q) && (!grad_w || aligned(grad_w)) && (!w_latent || aligned(w_latent)))
        vec = uint64_t(n) * esz / 16;
    if (vec) {
        const unsigned grid = grid_for(vec, 256, 8);
        if (dtype == E8Q_BF16)
            launch(ste_bf16_kernel, dim3(grid), dim3(256), 0, s,
                               static_cast<const uint4*>(grad_q), static_cast<uint4*>(grad_w),
                               static_cast<uint4*>(w_latent), lr, vec);
        else
            launch(ste_f32_kernel, dim3(grid), dim3(256), 0, s,
                               static_cast<const float4*>(grad_q), static_cast<float4*>(grad_w),
                               static_cast<float4*>(w_latent), lr, vec);
    }
    const uint64_t done = vec * 16 / esz;
    if (done < uint64_t(n)) {
        const uint64_t rest = uint64_t(n) - done;
        const unsigned grid = grid_for(rest, 256, 4);
        launch(ste_tail_kernel, dim3(grid), dim3(256), 0, s, grad_q, grad_w, w_latent, lr,
                           int(dtype == E8Q_BF16), done, uint64_t(n));
    }
    return launch_status();
}
