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
//     row error is sum (fl64(kappa_b * v) - s_k z)^2 over the row in a fixed
//     order (group sums pairwise; group g into partial g mod 64 in increasing
//     g; a butterfly over the 64 partials); the smallest error wins, NaN
//     counts as +inf, ties go to the smaller k, a candidate with an invalid
//     scale (the projection's bad-row rule) has error +inf.
//
// One wave per row.  The un-normalized transform v of the weights is computed
// once (e8q_rotate.hpp) into the workspace.  Per candidate, the lanes stride
// over the row's groups: the nearest E8 point and, for points inside the core,
// the group error go to LDS; groups outside the core are listed (in group
// order) and then searched 64 at a time, one per lane, over the core points,
// whose float64 coordinates are read as wave-uniform values.  The row error is
// then summed from LDS in the fixed order.
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"
#include "e8q_rotate.hpp"

namespace e8q {

constexpr int kPtqWaves = 2;   // waves (rows) per block

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
    const uint16_t* tab;
    RankParams rp;
    float* scale_out;
    int32_t* choice_out;
    double* err_out;           // [rows_total, n_alpha] or null
    uint16_t* core_idx;
    int8_t* two_z;
    uint32_t* status;
};

// Orders this wave's LDS accesses across lanes (a lane reads what another
// lane of the same wave wrote).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// One candidate scale over one row.  Returns the row error (valid on every
// lane); with WRITE the points of the row are stored.
template <bool WRITE>
__device__ double row_pass(const PtqArgs& a, uint32_t row, float s, float c, double* s_e, uint16_t* s_list,
                           uint32_t& flags) {
    const uint32_t lane = threadIdx.x & 63u;
    const float* vrow = a.v + uint64_t(row) * a.cols;
    const double k64 = double(a.kappa), s64 = double(s);
    const uint64_t gbase = uint64_t(row) * a.gpr;
    uint32_t nlist = 0;
    for (uint32_t g0 = 0; g0 < a.gpr; g0 += kWave) {
        const uint32_t g = g0 + lane;
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
                if (WRITE) flags |= inv;
            } else {
                nearest_e8(x, t);
            }
            outside = norm_u32(t) > uint32_t(a.core_bound);
            if (!outside) {
                s_e[g] = group_error(v, t, k64, s64);
                if constexpr (WRITE) {
                    uint32_t f8 = 0;
                    *reinterpret_cast<uint2*>(a.two_z + (gbase + g) * 8) = pack_i8x8(t, f8);
                    a.core_idx[gbase + g] = uint16_t(core_rank(t, a.tab, a.rp));
                }
            }
        }
        const uint64_t m = __ballot(outside);
        if (outside) s_list[nlist + __popcll(m & ((1ull << lane) - 1ull))] = uint16_t(g);
        nlist += uint32_t(__popcll(m));
    }
    wave_sync();
    // groups outside the core: exhaustive search, one group per lane
    for (uint32_t j0 = 0; j0 < nlist; j0 += kWave) {
        const uint32_t j = j0 + lane;
        const bool act = j < nlist;
        const uint32_t g = act ? uint32_t(s_list[j]) : 0u;
        float v[8];
        load_v(vrow, g, v);
        double x64[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x64[i] = double(v[i] * c);
        double best = -__builtin_inf();
        uint32_t bi = 0;
        // the candidate is the same on every lane: read it through the constant
        // address space so that it comes in with scalar loads
        typedef const __attribute__((address_space(4))) double* const_dptr;
        const const_dptr pts = (const_dptr)(uintptr_t)a.pts64;
#pragma unroll 2
        for (uint32_t p = 0; p < a.npts; ++p) {
            const const_dptr tp = pts + uint64_t(p) * 9;
            double q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = x64[i] * tp[i];
            const double key = (((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]))) - tp[8];
            if (key > best) {
                best = key;
                bi = p;
            }
        }
        if (act) {
            const double* tp = a.pts64 + uint64_t(bi) * 9;
            int t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = int(tp[i]);
            s_e[g] = group_error(v, t, k64, s64);
            if constexpr (WRITE) {
                uint32_t f8 = 0;
                *reinterpret_cast<uint2*>(a.two_z + (gbase + g) * 8) = pack_i8x8(t, f8);
                a.core_idx[gbase + g] = uint16_t(bi);
            }
        }
    }
    wave_sync();
    // the row error in the fixed order
    double acc = 0.0;
    for (uint32_t g = lane; g < a.gpr; g += kWave) acc = acc + s_e[g];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
    wave_sync();   // the buffers are reused by the next candidate
    return acc;
}

__global__ __launch_bounds__(kPtqWaves * kWave) void ptq_kernel(PtqArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t wv = threadIdx.x >> 6;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t row = blockIdx.x * kPtqWaves + wv;
    if (row >= a.rows_total) return;   // whole wave leaves; no block barrier below
    double* s_e = reinterpret_cast<double*>(s_dyn) + size_t(wv) * a.gpr;
    uint16_t* s_list = reinterpret_cast<uint16_t*>(reinterpret_cast<double*>(s_dyn) + size_t(kPtqWaves) * a.gpr) +
                       size_t(wv) * a.gpr;
    const float s0 = a.s0[row];
    uint32_t flags = 0;
    double best = __builtin_inf();
    int32_t kbest = 0;
    for (int32_t k = 0; k < a.n_alpha; ++k) {
        const float s = a.alphas[k] * s0;
        bool bad;
        const float c = row_coef(s, a.kappa, bad);
        double e = __builtin_inf();
        if (!bad) e = row_pass<false>(a, row, s, c, s_e, s_list, flags);
        if (a.err_out && lane == 0) a.err_out[uint64_t(row) * uint32_t(a.n_alpha) + uint32_t(k)] = e;
        const double key = e != e ? __builtin_inf() : e;
        if (key < best) {
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
        for (uint32_t g = lane; g < a.gpr; g += kWave) {
            *reinterpret_cast<uint2*>(a.two_z + (uint64_t(row) * a.gpr + g) * 8) = make_uint2(0u, 0u);
            a.core_idx[uint64_t(row) * a.gpr + g] = zero_idx;
        }
        flags |= E8Q_STATUS_BAD_SCALE;
    } else {
        (void)row_pass<true>(a, row, s, c, s_e, s_list, flags);
    }
    if (lane == 0) {
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
    const size_t lds = size_t(kPtqWaves) * gpr * (8 + 2);
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
    a.npts = uint32_t(tab->host.size);
    a.tab = tab->dptr;
    a.rp = tab->host.p;
    a.scale_out = scale_out;
    a.choice_out = choice_out;
    a.err_out = err_out;
    a.core_idx = core_idx_out;
    a.two_z = two_z_out;
    a.status = status_dev;
    const unsigned grid = unsigned((rows_total + kPtqWaves - 1) / kPtqWaves);
    hipLaunchKernelGGL(ptq_kernel, dim3(grid), dim3(kPtqWaves * kWave), lds, s, a);
    return launch_status();
}
