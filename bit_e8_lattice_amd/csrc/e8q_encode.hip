// e8q_encode_core_escape: export encoding into 16-bit core indices plus
// compacted exact escape records.
//
// E8-QAT keeps the final lattice points exactly: a 2-bit-per-weight core index
// per group and a sparse 20-byte record for each group outside the finite
// core (abstract; Figure 2(c) and Figure 6(c) captions; Table 10).
//
// One pass over the weights: each 256-thread block claims tiles of 2048
// consecutive groups in increasing order (a device-wide counter), computes
// every lattice point and core index of the tile, counts its escapes (wave
// ballots, then a block scan), and resolves the tile's output offset with a
// decoupled look-back over the per-tile status words (aggregate / inclusive
// prefix, packed with their flag into one 64-bit word).  Escape records thus
// land in ascending group order whatever the scheduling.
#include <map>
#include <mutex>
#include <utility>

#include "e8q_core_table.hpp"
#include "e8q_device.hpp"
#include "e8q_host.hpp"

namespace e8q {

constexpr int kItems = 8;                          // groups per thread per tile
constexpr int kBlock = 256;
constexpr uint32_t kTileGroups = kItems * kBlock;  // 2048
constexpr uint64_t kFlagA = 1ull << 62;            // aggregate published
constexpr uint64_t kFlagP = 2ull << 62;            // inclusive prefix published
constexpr uint64_t kValMask = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr size_t kWsHeader = 256;

struct EncodeArgs {
    const void* w;
    uint32_t groups;
    uint32_t gpr;
    FastDiv gpr_div;
    FastDiv gpb_div;
    const float* scale;
    const int8_t* signs;
    float kappa;
    int core_bound;
    const uint16_t* tab;
    RankParams rp;
    uint16_t* core_idx;
    e8q_escape_t* esc;
    uint64_t esc_cap;
    unsigned long long* esc_count;
    int8_t* two_z;
    uint32_t* tile_counter;
    unsigned long long* tile_status;
    uint32_t num_tiles;
    uint32_t* status;
};

__device__ __forceinline__ uint32_t core_rank(const int (&t)[8], const uint16_t* tab, const RankParams& p) {
    const int c = t[0] & 1;
    const int tm = c ? p.tm[1] : p.tm[0];
    const uint32_t base = uint32_t(tm + 1);
    uint32_t ha = 0, hb = 0;
    int na = 0, sa = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ha = ha * base + uint32_t((t[i] + tm) >> 1);
        hb = hb * base + uint32_t((t[4 + i] + tm) >> 1);
        na += t[i] * t[i];
        sa += t[i];
    }
    const uint32_t f = tab[(c ? p.off_f[1] : p.off_f[0]) + ha];
    const uint32_t nh = c ? p.nh[1] : p.nh[0];
    const uint32_t g = tab[(c ? p.off_g[1] : p.off_g[0]) + uint32_t((na >> 2) * 2 + ((sa >> 1) & 1)) * nh + hb];
    return f + g;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
    const uint32_t lo = __shfl_xor(uint32_t(v), m, 64);
    const uint32_t hi = __shfl_xor(uint32_t(v >> 32), m, 64);
    return (uint64_t(hi) << 32) | lo;
}

__global__ void encode_init_kernel(uint32_t* counter, unsigned long long* tile_status, uint32_t num_tiles,
                                   unsigned long long* esc_count, uint32_t batch) {
    const uint32_t i0 = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t stride = gridDim.x * blockDim.x;
    if (i0 == 0) *counter = 0u;
    for (uint32_t i = i0; i < num_tiles; i += stride) tile_status[i] = 0ull;
    for (uint32_t i = i0; i < batch; i += stride) esc_count[i] = 0ull;
}

template <typename WT, int HB, bool LDS_TAB>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeArgs a) {
    extern __shared__ uint16_t s_tab[];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_cnt[kItems][kBlock / kWave];
    __shared__ unsigned long long s_total;
    __shared__ unsigned long long s_excl;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = __lane_id();
    const uint32_t wv = tid / kWave;
    const uint16_t* tab = a.tab;
    if constexpr (LDS_TAB) {
        for (uint32_t i = tid; i < a.rp.entries; i += kBlock) s_tab[i] = a.tab[i];
        tab = s_tab;
    }

    for (;;) {
        __syncthreads();
        if (tid == 0) s_tile = atomicAdd(a.tile_counter, 1u);
        __syncthreads();
        const uint32_t tile = s_tile;
        if (tile >= a.num_tiles) break;

        uint32_t esc_bits = 0;
        uint32_t in_wave[kItems];
        uint32_t rec[kItems][4];
        uint32_t flags = 0;

#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const uint32_t g = tile * kTileGroups + uint32_t(j) * kBlock + tid;
            const bool live = g < a.groups;
            float v[8];
            if (live) {
                load_group(reinterpret_cast<const WT*>(a.w), g, v);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.0f;
            }
            const uint32_t row = live ? fdiv(g, a.gpr_div) : 0u;
            if constexpr (HB > 0) {
                const uint32_t col0 = (g - row * a.gpr) * 8u;
                if (live) apply_signs(a.signs, col0, v);
                fwht_group<HB>(v, lane);
            }
            bool bad;
            const float c = row_coef(a.scale[row], a.kappa, bad);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = v[i] * c;
            int t[8];
            uint32_t inv = bad ? uint32_t(E8Q_STATUS_BAD_SCALE) : group_invalid_bits(x);
            if (inv) {
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = 0;
                if (live) flags |= inv;
            } else {
                nearest_e8(x, t);
            }
            uint32_t norm = 0;   // <= 8 * 16386^2 < 2^32
#pragma unroll
            for (int i = 0; i < 8; ++i) norm += uint32_t(t[i] * t[i]);
            const bool escaped = live && norm > uint32_t(a.core_bound);
            if (live) a.core_idx[g] = escaped ? uint16_t(0xFFFF) : uint16_t(core_rank(t, tab, a.rp));
            if (a.two_z) {
                uint32_t f8 = 0;
                const uint2 p = pack_i8x8(t, f8);
                if (live) {
                    *reinterpret_cast<uint2*>(a.two_z + uint64_t(g) * 8) = p;
                    flags |= f8;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rec[j][i] = (uint32_t(t[2 * i]) & 0xFFFFu) | (uint32_t(t[2 * i + 1]) << 16);
            const uint64_t mask = __ballot(escaped);
            in_wave[j] = __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
            if (lane == 0) s_cnt[j][wv] = uint32_t(__popcll(mask));
            esc_bits |= escaped ? (1u << j) : 0u;
            if (mask) {
                const uint32_t b = live ? fdiv(g, a.gpb_div) : 0u;
                const uint32_t b0 = __shfl(b, 0, 64);
                const bool uniform = __ballot(live && b != b0) == 0;
                if (uniform) {
                    if (lane == 0) atomicAdd(a.esc_count + b0, (unsigned long long)__popcll(mask));
                } else if (escaped) {
                    atomicAdd(a.esc_count + b, 1ull);
                }
            }
        }
        flush_status(flags, a.status);
        __syncthreads();

        // Exclusive offsets of every (item, wave) inside the tile, item-major:
        // that is ascending group order.
        if (tid == 0) {
            uint32_t run = 0;
            for (int j = 0; j < kItems; ++j)
                for (int k = 0; k < kBlock / kWave; ++k) {
                    const uint32_t c = s_cnt[j][k];
                    s_cnt[j][k] = run;
                    run += c;
                }
            s_total = run;
        }
        __syncthreads();

        // Decoupled look-back (first wave).
        if (wv == 0) {
            const unsigned long long total = s_total;
            unsigned long long excl = 0;
            bool timeout = false;
            if (tile == 0) {
                if (lane == 0)
                    __hip_atomic_store(a.tile_status, kFlagP | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                if (lane == 0)
                    __hip_atomic_store(a.tile_status + tile, kFlagA | total, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                int64_t j = int64_t(tile) - 1;
                uint32_t spins = 0;
                for (;;) {
                    const int64_t idx = j - int64_t(lane);
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
                    j -= 64;
                }
                if (lane == 0)
                    __hip_atomic_store(a.tile_status + tile, kFlagP | ((excl + total) & kValMask), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            if (lane == 0) {
                s_excl = excl;
                if (timeout) atomicOr(a.status, uint32_t(E8Q_STATUS_LOOKBACK_TIMEOUT));
            }
        }
        __syncthreads();

        uint32_t oflags = 0;
        if (esc_bits) {
            const unsigned long long excl = s_excl;
#pragma unroll
            for (int j = 0; j < kItems; ++j) {
                if (esc_bits & (1u << j)) {
                    const uint32_t g = tile * kTileGroups + uint32_t(j) * kBlock + tid;
                    const unsigned long long pos = excl + s_cnt[j][wv] + in_wave[j];
                    if (pos < a.esc_cap) {
                        const uint32_t grp = g - fdiv(g, a.gpb_div) * a.gpb_div.d;
                        uint32_t* dst = reinterpret_cast<uint32_t*>(a.esc + pos);
                        dst[0] = grp;
                        dst[1] = rec[j][0];
                        dst[2] = rec[j][1];
                        dst[3] = rec[j][2];
                        dst[4] = rec[j][3];
                    } else {
                        oflags |= E8Q_STATUS_ESC_OVERFLOW;
                    }
                }
            }
        }
        flush_status(oflags, a.status);
    }
}

// ------------------------------------------------------------------ host

namespace {

struct DevTable {
    uint16_t* dptr = nullptr;
    CoreTable host;
};

std::mutex g_tab_mu;
std::map<std::pair<int, int>, DevTable>* g_tabs = nullptr;

// Rank table for (current device, bound), uploaded once and kept for the
// life of the process.
const DevTable* get_table(int32_t bound, e8q_status_t& err) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_tab_mu);
    if (!g_tabs) g_tabs = new std::map<std::pair<int, int>, DevTable>();
    auto key = std::make_pair(dev, int(bound));
    auto it = g_tabs->find(key);
    if (it != g_tabs->end()) return &it->second;
    DevTable t;
    if (!build_core_table(bound, t.host)) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    const size_t bytes = t.host.data.size() * sizeof(uint16_t);
    if (hipMalloc(&t.dptr, bytes) != hipSuccess) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    if (hipMemcpy(t.dptr, t.host.data.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    auto res = g_tabs->emplace(key, std::move(t));
    return &res.first->second;
}

uint32_t tiles_for(int64_t batch, int64_t rows, int64_t cols) {
    const uint64_t groups = uint64_t(batch) * uint64_t(rows) * uint64_t(cols / 8);
    return uint32_t((groups + kTileGroups - 1) / kTileGroups);
}

template <typename WT, bool LDS>
void launch_encode(int hb, const EncodeArgs& a, unsigned grid, size_t lds, hipStream_t st) {
    switch (hb) {
        case 0: hipLaunchKernelGGL((encode_kernel<WT, 0, LDS>), dim3(grid), dim3(kBlock), lds, st, a); break;
        case 8: hipLaunchKernelGGL((encode_kernel<WT, 8, LDS>), dim3(grid), dim3(kBlock), lds, st, a); break;
        case 16: hipLaunchKernelGGL((encode_kernel<WT, 16, LDS>), dim3(grid), dim3(kBlock), lds, st, a); break;
        case 32: hipLaunchKernelGGL((encode_kernel<WT, 32, LDS>), dim3(grid), dim3(kBlock), lds, st, a); break;
        case 64: hipLaunchKernelGGL((encode_kernel<WT, 64, LDS>), dim3(grid), dim3(kBlock), lds, st, a); break;
        case 128: hipLaunchKernelGGL((encode_kernel<WT, 128, LDS>), dim3(grid), dim3(kBlock), lds, st, a); break;
        default: break;
    }
}

}  // namespace

int64_t core_size_host(int32_t bound) {
    CoreTable t;
    if (!build_core_table(bound, t)) return -1;
    return t.size;
}

}  // namespace e8q

extern "C" size_t e8q_encode_workspace_size(int64_t batch, int64_t rows, int64_t cols) {
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 8) return 0;
    return e8q::kWsHeader + sizeof(unsigned long long) * size_t(e8q::tiles_for(batch, rows, cols));
}

extern "C" e8q_status_t e8q_encode_core_escape(const void* w, e8q_dtype_t w_dtype, int64_t batch,
                                               int64_t rows, int64_t cols, const float* row_scale,
                                               const int8_t* signs, int32_t had_block,
                                               int32_t core_bound, uint16_t* core_idx_out,
                                               e8q_escape_t* esc_out, int64_t esc_capacity,
                                               int64_t* esc_count_out, int8_t* two_z_out,
                                               void* workspace, size_t workspace_bytes,
                                               uint32_t* status_dev, void* stream) {
    using namespace e8q;
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
        if (hb > 128) return E8Q_ERR_UNSUPPORTED;   // wider blocks: not in this build
    }
    const DevTable* tab = get_table(core_bound, st);
    if (!tab) return st;

    const uint32_t gpr = uint32_t(cols / 8);
    EncodeArgs a;
    a.w = w;
    a.groups = uint32_t(uint64_t(batch) * uint64_t(rows) * gpr);
    a.gpr = gpr;
    a.gpr_div = make_fastdiv(gpr);
    a.gpb_div = make_fastdiv(uint32_t(uint64_t(rows) * gpr));
    a.scale = row_scale;
    a.signs = signs;
    a.kappa = kappa_for(hb);
    a.core_bound = core_bound;
    a.tab = tab->dptr;
    a.rp = tab->host.p;
    a.core_idx = core_idx_out;
    a.esc = esc_out;
    a.esc_cap = uint64_t(esc_capacity);
    a.esc_count = reinterpret_cast<unsigned long long*>(esc_count_out);
    a.two_z = two_z_out;
    a.tile_counter = reinterpret_cast<uint32_t*>(workspace);
    a.tile_status = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + kWsHeader);
    a.num_tiles = tiles_for(batch, rows, cols);
    a.status = status_dev;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint32_t init_items = a.num_tiles > uint32_t(batch) ? a.num_tiles : uint32_t(batch);
    hipLaunchKernelGGL(encode_init_kernel, dim3(grid_for(init_items, 256, 4)), dim3(256), 0, s,
                       a.tile_counter, a.tile_status, a.num_tiles, a.esc_count, uint32_t(batch));
    const unsigned grid = grid_for(a.num_tiles, 1, 4);
    const bool lds = core_bound <= kLdsTableMaxBound;
    const size_t lds_bytes = lds ? size_t(a.rp.entries) * sizeof(uint16_t) : 0;
    if (w_dtype == E8Q_BF16) {
        if (lds) launch_encode<uint16_t, true>(hb, a, grid, lds_bytes, s);
        else launch_encode<uint16_t, false>(hb, a, grid, 0, s);
    } else {
        if (lds) launch_encode<float, true>(hb, a, grid, lds_bytes, s);
        else launch_encode<float, false>(hb, a, grid, 0, s);
    }
    return launch_status();
}
