// e8q_ste_backward: identity straight-through estimator, optionally fused with
// the SGD step on the latent weights.
//
// E8-QAT trains through the projection with an identity STE (Figure 2(b)
// caption), so dL/dw = dL/dq bit for bit; latents are BF16 (Table 4).  The
// fused update reads g and w once and writes w once: 16-byte vector accesses,
// a pure HBM stream.
#include "e8q_device.hpp"
#include "e8q_host.hpp"

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

}  // namespace e8q

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
            hipLaunchKernelGGL(ste_bf16_kernel, dim3(grid), dim3(256), 0, s,
                               static_cast<const uint4*>(grad_q), static_cast<uint4*>(grad_w),
                               static_cast<uint4*>(w_latent), lr, vec);
        else
            hipLaunchKernelGGL(ste_f32_kernel, dim3(grid), dim3(256), 0, s,
                               static_cast<const float4*>(grad_q), static_cast<float4*>(grad_w),
                               static_cast<float4*>(w_latent), lr, vec);
    }
    const uint64_t done = vec * 16 / esz;
    if (done < uint64_t(n)) {
        const uint64_t rest = uint64_t(n) - done;
        const unsigned grid = grid_for(rest, 256, 4);
        hipLaunchKernelGGL(ste_tail_kernel, dim3(grid), dim3(256), 0, s, grad_q, grad_w, w_latent, lr,
                           int(dtype == E8Q_BF16), done, uint64_t(n));
    }
    return launch_status();
}
