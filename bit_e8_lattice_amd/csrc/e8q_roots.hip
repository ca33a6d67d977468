// e8q_pack_escapes / e8q_unpack_escapes: escape records as a core index plus
// a root of E8.
//
// E8-QAT checks that every escaped group of its artifact is a core point plus
// one root (Table 3: single-root membership), which is what makes a record of
// a core index and a root enough.  The pages leave the choice of root open;
// here it is the first root, in lexicographic order of 2r, that brings the
// point into the core.  A point no root brings into the core keeps its full
// 20-byte record in a second list.
//
// Both directions are one pass over the records in blocks of 1024 (the root
// search is a loop over the 240 roots held in LDS as int16 pairs, the test
// ||t - 2r||^2 <= B taken as 2 t.(2r) >= ||t||^2 + 8 - B with four packed
// int16 dot products per root; records are sparse), then
// an exclusive scan of the per-block counts of wide records, then a pass that
// places the wide records in record order.
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"

namespace e8q {

constexpr int kRootThreads = 256;
constexpr int kRootPer = 4;                           // records per thread
constexpr int kRootBlock = kRootThreads * kRootPer;   // records per block

struct RootArgs {
    const uint32_t* esc;        // 20-byte records as words (pack input / unpack wide list)
    uint32_t* packed;           // 8-byte packed records as words
    uint32_t* wide;             // 20-byte records as words (pack output / unpack output)
    uint64_t n;
    uint64_t wide_cap;          // pack: capacity of the wide list; unpack: records in it
    const uint32_t* roots;
    const uint16_t* tab;
    RankParams rp;
    uint32_t npts;
    const uint32_t* pts;
    int core_bound;
    uint64_t* block_counts;     // workspace
    int64_t* wide_count;        // pack output
    uint32_t* status;
};

__device__ __forceinline__ void bytes_to_ints(uint32_t w0, uint32_t w1, int (&t)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        t[i] = int((w0 >> (8 * i)) & 0xFFu) - 64;
        t[4 + i] = int((w1 >> (8 * i)) & 0xFFu) - 64;
    }
}

// Block-wide exclusive scan of one count per thread; returns the prefix and
// writes the block total to *total (every thread).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_scan, uint32_t& total) {
    const uint32_t tid = threadIdx.x;
    s_scan[tid] = v;
    __syncthreads();
    for (uint32_t d = 1; d < uint32_t(kRootThreads); d <<= 1) {
        const uint32_t add = tid >= d ? s_scan[tid - d] : 0u;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
    }
    total = s_scan[kRootThreads - 1];
    const uint32_t incl = s_scan[tid];
    __syncthreads();
    return incl - v;
}

// Pack: root search and core index per record, packed record out, count of
// records that need a wide record per block.
typedef short rt_short2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kRootThreads) void pack_kernel(RootArgs a) {
    // the roots as 2r in int16 pairs (four words per root)
    __shared__ uint32_t s_r16[960];
    __shared__ uint32_t s_scan[kRootThreads];
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < 960u; i += kRootThreads) {
        const uint32_t w = a.roots[2u * (i >> 2) + ((i >> 1) & 1u)];
        const uint32_t sh = 16u * (i & 1u);   // bytes 2i', 2i'+1 of the word pair
        const int lo = int((w >> sh) & 0xFFu) - 64, hi = int((w >> (sh + 8u)) & 0xFFu) - 64;
        s_r16[i] = (uint32_t(lo) & 0xFFFFu) | (uint32_t(hi) << 16);
    }
    __syncthreads();
    const uint64_t base = uint64_t(blockIdx.x) * kRootBlock + uint64_t(tid) * kRootPer;
    uint32_t nwide = 0;
    for (int k = 0; k < kRootPer; ++k) {
        const uint64_t i = base + k;
        if (i >= a.n) break;
        const uint32_t* r = a.esc + i * 5;
        // 2z as int16 pairs, as the record stores it
        const uint32_t w[4] = {r[1], r[2], r[3], r[4]};
        int t[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            t[2 * q] = int(int16_t(uint16_t(w[q] & 0xFFFFu)));
            t[2 * q + 1] = int(int16_t(uint16_t(w[q] >> 16)));
        }
        uint32_t nt = 0;   // ||t||^2 < 8 * 16386^2 < 2^32
#pragma unroll
        for (int q = 0; q < 8; ++q) nt += uint32_t(t[q] * t[q]);
        // ||t - 2r||^2 = ||t||^2 - 2 t.(2r) + 8 <= B  <=>  2 t.(2r) >= ||t||^2 + 8 - B;
        // |t.(2r)| <= 8 * 16386 (2r is (+-2, +-2, 0, ...) or (+-1, ...)), so a
        // larger threshold admits no root
        const int64_t need = int64_t(nt) + 8 - int64_t(a.core_bound);
        uint32_t root = 0xFFu, core = 0xFFFFu;
        if (need <= 2 * 131088) {
            const int th = int(need);
            // eight roots per step (independent dot products), the first hit
            // of the step from its bit mask
            for (uint32_t j0 = 0; j0 < 240u; j0 += 8u) {
                uint32_t hits = 0;
#pragma unroll
                for (uint32_t k = 0; k < 8u; ++k) {
                    const uint32_t* rr = s_r16 + 4u * (j0 + k);
                    int dot = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        dot = __builtin_amdgcn_sdot2(__builtin_bit_cast(rt_short2, w[q]),
                                                     __builtin_bit_cast(rt_short2, rr[q]), dot, false);
                    hits |= (2 * dot >= th ? 1u : 0u) << k;
                }
                if (hits != 0u) {
                    const uint32_t j = j0 + uint32_t(__builtin_ctz(hits));
                    const uint32_t* rr = s_r16 + 4u * j;
                    int c[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        c[2 * q] = t[2 * q] - int(int16_t(uint16_t(rr[q] & 0xFFFFu)));
                        c[2 * q + 1] = t[2 * q + 1] - int(int16_t(uint16_t(rr[q] >> 16)));
                    }
                    root = j;
                    core = core_rank(c, a.tab, a.rp);
                    break;
                }
            }
        }
        a.packed[2 * i] = r[0];
        a.packed[2 * i + 1] = core | (root << 16);
        nwide += root == 0xFFu ? 1u : 0u;
    }
    uint32_t total;
    block_exclusive_scan(nwide, s_scan, total);
    if (tid == 0) a.block_counts[blockIdx.x] = total;
}

// Unpack, first pass: count packed records that refer to the wide list.
__global__ __launch_bounds__(kRootThreads) void unpack_count_kernel(RootArgs a) {
    __shared__ uint32_t s_scan[kRootThreads];
    const uint32_t tid = threadIdx.x;
    const uint64_t base = uint64_t(blockIdx.x) * kRootBlock + uint64_t(tid) * kRootPer;
    uint32_t nwide = 0;
    for (int k = 0; k < kRootPer; ++k) {
        const uint64_t i = base + k;
        if (i >= a.n) break;
        nwide += ((a.packed[2 * i + 1] >> 16) & 0xFFu) == 0xFFu ? 1u : 0u;
    }
    uint32_t total;
    block_exclusive_scan(nwide, s_scan, total);
    if (tid == 0) a.block_counts[blockIdx.x] = total;
}

// Exclusive scan of the block counts in place (one block); the total goes to
// *total_out when given.
__global__ __launch_bounds__(1024) void scan_counts_kernel(uint64_t* counts, uint64_t nblocks, int64_t* total_out) {
    __shared__ uint64_t part[1024];
    const uint32_t tid = threadIdx.x;
    const uint64_t chunk = (nblocks + 1023u) / 1024u;
    const uint64_t lo = min(uint64_t(tid) * chunk, nblocks), hi = min(lo + chunk, nblocks);
    uint64_t sum = 0;
    for (uint64_t i = lo; i < hi; ++i) sum += counts[i];
    part[tid] = sum;
    __syncthreads();
    for (uint32_t d = 1; d < 1024u; d <<= 1) {
        const uint64_t v = tid >= d ? part[tid - d] : 0ull;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    uint64_t run = part[tid] - sum;
    for (uint64_t i = lo; i < hi; ++i) {
        const uint64_t c = counts[i];
        counts[i] = run;
        run += c;
    }
    if (tid == 1023u && total_out) *total_out = int64_t(part[1023]);
}

// Second pass.  Pack: copy the records without a root to the wide list.
// Unpack: rebuild every 20-byte record.
template <bool PACK>
__global__ __launch_bounds__(kRootThreads) void place_kernel(RootArgs a) {
    __shared__ uint32_t s_scan[kRootThreads];
    __shared__ uint32_t s_roots[480];
    const uint32_t tid = threadIdx.x;
    if constexpr (!PACK) {
        for (uint32_t i = tid; i < 480u; i += kRootThreads) s_roots[i] = a.roots[i];
    }
    const uint64_t base = uint64_t(blockIdx.x) * kRootBlock + uint64_t(tid) * kRootPer;
    uint32_t nwide = 0;
    for (int k = 0; k < kRootPer; ++k) {
        const uint64_t i = base + k;
        if (i >= a.n) break;
        nwide += ((a.packed[2 * i + 1] >> 16) & 0xFFu) == 0xFFu ? 1u : 0u;
    }
    uint32_t total;
    const uint64_t pos0 = a.block_counts[blockIdx.x] + block_exclusive_scan(nwide, s_scan, total);
    uint32_t flags = 0;
    uint64_t pos = pos0;
    for (int k = 0; k < kRootPer; ++k) {
        const uint64_t i = base + k;
        if (i >= a.n) break;
        const uint32_t w1 = a.packed[2 * i + 1];
        const uint32_t root = (w1 >> 16) & 0xFFu, core = w1 & 0xFFFFu;
        if constexpr (PACK) {
            if (root == 0xFFu) {
                if (pos < a.wide_cap) {
#pragma unroll
                    for (int q = 0; q < 5; ++q) a.wide[pos * 5 + q] = a.esc[i * 5 + q];
                } else {
                    flags |= E8Q_STATUS_ESC_OVERFLOW;
                }
                ++pos;
            }
        } else {
            uint32_t* o = a.wide + i * 5;   // unpack output
            o[0] = a.packed[2 * i];
            if (root == 0xFFu) {
                if (pos < a.wide_cap) {
#pragma unroll
                    for (int q = 1; q < 5; ++q) o[q] = a.esc[pos * 5 + q];
                } else {
                    flags |= E8Q_STATUS_ESC_MISSING;
#pragma unroll
                    for (int q = 1; q < 5; ++q) o[q] = 0u;
                }
                ++pos;
            } else {
                int t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (root < 240u && core < a.npts) {
                    int c[8], rr[8];
                    bytes_to_ints(a.pts[2 * core], a.pts[2 * core + 1], c);
                    bytes_to_ints(s_roots[2 * root], s_roots[2 * root + 1], rr);
#pragma unroll
                    for (int q = 0; q < 8; ++q) t[q] = c[q] + rr[q];
                } else {
                    flags |= E8Q_STATUS_BAD_INDEX;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[1 + q] = (uint32_t(t[2 * q]) & 0xFFFFu) | (uint32_t(t[2 * q + 1]) << 16);
            }
        }
    }
    flush_status(flags, a.status);
}

static size_t roots_ws_bytes(int64_t n) {
    const uint64_t nb = (uint64_t(n) + kRootBlock - 1) / kRootBlock;
    return (size_t(nb > 0 ? nb : 1) * 8 + 255) & ~size_t(255);
}

static e8q_status_t prepare(RootArgs& a, int64_t n, int32_t core_bound, void* workspace, size_t workspace_bytes,
                            uint32_t* status_dev) {
    if (n < 0 || core_bound < 0 || core_bound > 40 || !status_dev || !workspace) return E8Q_ERR_INVALID;
    if (workspace_bytes < roots_ws_bytes(n) || (reinterpret_cast<uintptr_t>(workspace) & 7u)) return E8Q_ERR_INVALID;
    if ((uint64_t(n) + kRootBlock - 1) / kRootBlock >= (uint64_t(1) << 31)) return E8Q_ERR_UNSUPPORTED;
    e8q_status_t err = E8Q_OK;
    const DevTable* tab = get_table(core_bound, err);
    if (!tab) return err;
    a.n = uint64_t(n);
    a.roots = tab->droots;
    a.tab = tab->dptr;
    a.rp = tab->p;
    a.npts = uint32_t(tab->size);
    a.pts = tab->dpoints;
    a.core_bound = core_bound;
    a.block_counts = static_cast<uint64_t*>(workspace);
    a.status = status_dev;
    return E8Q_OK;
}

}  // namespace e8q

extern "C" size_t e8q_pack_workspace_size(int64_t n) {
    if (n < 0) return 0;
    return e8q::roots_ws_bytes(n);
}

extern "C" e8q_status_t e8q_pack_escapes(const e8q_escape_t* esc, int64_t n, int32_t core_bound,
                                         e8q_escape_packed_t* packed_out, e8q_escape_t* wide_out,
                                         int64_t wide_capacity, int64_t* wide_count_out, void* workspace,
                                         size_t workspace_bytes, uint32_t* status_dev, void* stream) {
    using namespace e8q;
    if (!wide_count_out || wide_capacity < 0 || (wide_capacity > 0 && !wide_out)) return E8Q_ERR_INVALID;
    if (n > 0 && (!esc || !packed_out)) return E8Q_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(esc) | reinterpret_cast<uintptr_t>(wide_out)) & 3u) return E8Q_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(packed_out) & 7u) return E8Q_ERR_INVALID;
    RootArgs a{};
    e8q_status_t st = prepare(a, n, core_bound, workspace, workspace_bytes, status_dev);
    if (st != E8Q_OK) return st;
    a.esc = reinterpret_cast<const uint32_t*>(esc);
    a.packed = reinterpret_cast<uint32_t*>(packed_out);
    a.wide = reinterpret_cast<uint32_t*>(wide_out);
    a.wide_cap = uint64_t(wide_capacity);
    a.wide_count = wide_count_out;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint64_t nb = (uint64_t(n) + kRootBlock - 1) / kRootBlock;
    if (nb == 0) {
        launch(scan_counts_kernel, dim3(1), dim3(1024), 0, s, a.block_counts, uint64_t(0),
                           wide_count_out);
        return launch_status();
    }
    launch(pack_kernel, dim3(unsigned(nb)), dim3(kRootThreads), 0, s, a);
    launch(scan_counts_kernel, dim3(1), dim3(1024), 0, s, a.block_counts, nb, wide_count_out);
    launch(place_kernel<true>, dim3(unsigned(nb)), dim3(kRootThreads), 0, s, a);
    return launch_status();
}

extern "C" e8q_status_t e8q_unpack_escapes(const e8q_escape_packed_t* packed, int64_t n, const e8q_escape_t* wide,
                                           int64_t wide_count, int32_t core_bound, e8q_escape_t* esc_out,
                                           void* workspace, size_t workspace_bytes, uint32_t* status_dev,
                                           void* stream) {
    using namespace e8q;
    if (wide_count < 0 || (wide_count > 0 && !wide)) return E8Q_ERR_INVALID;
    if (n > 0 && (!packed || !esc_out)) return E8Q_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(esc_out) | reinterpret_cast<uintptr_t>(wide)) & 3u) return E8Q_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(packed) & 7u) return E8Q_ERR_INVALID;
    RootArgs a{};
    e8q_status_t st = prepare(a, n, core_bound, workspace, workspace_bytes, status_dev);
    if (st != E8Q_OK) return st;
    if (n == 0) return E8Q_OK;
    a.esc = reinterpret_cast<const uint32_t*>(wide);
    a.packed = const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(packed));
    a.wide = reinterpret_cast<uint32_t*>(esc_out);
    a.wide_cap = uint64_t(wide_count);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint64_t nb = (uint64_t(n) + kRootBlock - 1) / kRootBlock;
    launch(unpack_count_kernel, dim3(unsigned(nb)), dim3(kRootThreads), 0, s, a);
    launch(scan_counts_kernel, dim3(1), dim3(1024), 0, s, a.block_counts, nb, nullptr);
    launch(place_kernel<false>, dim3(unsigned(nb)), dim3(kRootThreads), 0, s, a);
    return launch_status();
}
