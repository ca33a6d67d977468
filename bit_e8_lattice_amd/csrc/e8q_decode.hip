// e8q_decode_core_escape: the exported form (16-bit core indices plus sparse
// escape records) back to lattice points, dequantized weights in the rotated
// basis, and restored weights in the original basis.
//
// E8-QAT keeps the selected lattice points exactly through its core indices
// and escape records (Figure 2(c) caption) and checks that its decoding paths
// agree on every core codeword (Table 3).  Decoding is a streaming map: each
// thread owns whole groups on the projection's tile layout (so the restore
// can reuse the lane-level inverse transform), a core index is one read of the
// point table (2z + 64 bytes, in LDS when it fits), and an escaped slot finds
// its record by binary search among the records of its batch item (records are
// in ascending group order).  A one-block prologue turns the per-batch counts
// into record offsets, clipped to the records actually present.
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"
#include "e8q_rotate.hpp"

namespace e8q {

struct DecodeArgs {
    const uint16_t* core_idx;
    const uint32_t* esc;          // records as 32-bit words, 5 per record
    const uint64_t* offsets;      // [batch + 1] record offsets (workspace)
    uint32_t groups;
    uint32_t gpr;
    uint32_t gpb;                 // groups per batch item
    FastDiv gpr_div;
    FastDiv gpb_div;
    const float* scale;
    float kappa;
    const int8_t* signs;
    uint32_t cols;
    const uint32_t* pts;          // point table (global copy)
    const uint32_t* h8;           // H_8 (2z) of the points as signed bytes
    uint32_t npts;
    int8_t* two_z;
    void* q;
    int q_bf16;
    void* w_hat;
    int w_hat_bf16;
    uint32_t* status;
    uint32_t num_tiles;
};

// Exclusive scan of the per-batch counts, each offset clipped to the capacity
// (negative counts count as 0).  One block of 1024 threads, any batch size.
__global__ __launch_bounds__(1024) void decode_offsets_kernel(const int64_t* counts, uint32_t batch,
                                                              uint64_t capacity, uint64_t* offsets) {
    __shared__ uint64_t part[1024];
    const uint32_t tid = threadIdx.x;
    const uint32_t chunk = (batch + 1023u) / 1024u;
    const uint32_t lo = min(tid * chunk, batch), hi = min(lo + chunk, batch);
    uint64_t sum = 0;
    for (uint32_t i = lo; i < hi; ++i) sum += counts[i] > 0 ? uint64_t(counts[i]) : 0ull;
    part[tid] = sum;
    __syncthreads();
    for (uint32_t d = 1; d < 1024u; d <<= 1) {
        const uint64_t v = tid >= d ? part[tid - d] : 0ull;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    uint64_t run = part[tid] - sum;
    for (uint32_t i = lo; i < hi; ++i) {
        offsets[i] = min(run, capacity);
        run += counts[i] > 0 ? uint64_t(counts[i]) : 0ull;
    }
    if (tid == 1023u) offsets[batch] = min(part[1023], capacity);
}

// 2z of an escaped slot from its record; false when there is none.  The
// records of a batch item hold increasing group indices below gpb, spread
// roughly evenly, so the first probes interpolate the position between the
// bracketing keys (each probe is a dependent load); then it halves.
__device__ __forceinline__ bool find_record(const uint32_t* esc, const uint64_t* offsets, uint32_t b, uint32_t gib,
                                            uint32_t gpb, int (&t)[8]) {
    uint64_t lo = offsets[b], hi = offsets[b + 1];
    uint32_t klo = 0u, khi = gpb;   // every key in [lo, hi) lies in [klo, khi) (sorted records)
    // at most 64 steps: the range never exceeds 2^64 records
    for (int it = 0; it < 64 && lo < hi; ++it) {
        uint64_t mid = lo + ((hi - lo) >> 1);
        if (it < 3 && gib >= klo && gib < khi && hi - lo <= 0xFFFFFFFFull) {
            // gib - klo < khi - klo, so off < hi - lo (no overflow: both factors < 2^32)
            mid = lo + uint64_t(gib - klo) * (hi - lo) / uint64_t(khi - klo);
        }
        const uint32_t key = esc[mid * 5];
        if (key == gib) {
            const uint32_t* r = esc + mid * 5 + 1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t wv = r[k];
                t[2 * k] = int(int16_t(uint16_t(wv & 0xFFFFu)));
                t[2 * k + 1] = int(int16_t(uint16_t(wv >> 16)));
            }
            return true;
        }
        if (key < gib) {
            lo = mid + 1;
            klo = key + 1u;
        } else {
            hi = mid;
            khi = key;
        }
    }
    return false;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short gm_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_rne_dec(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int HB, bool RESTORE, bool LDS_PTS>
__global__ __launch_bounds__(kBlock) void decode_kernel(DecodeArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wv = tid >> 6;
    const uint32_t smask_words = RESTORE ? a.cols / 2u : 0u;
    const uint32_t wide_words = (RESTORE && HB > 128) ? uint32_t(8 * kBlock) : 0u;
    uint32_t* s_smask = s_dyn;
    float* s_wide = reinterpret_cast<float*>(s_dyn + smask_words);
    // LDS tables: the points (2z + 64 bytes) when q or 2z is written, and for
    // the restore the in-lane part of the inverse transform of every point,
    // H_8 (2z) as signed bytes (|H_8 (2z)| <= 48 for any core), so that a core
    // group starts its transform at the cross-lane stages.
    const bool need_2z = a.q != nullptr || a.two_z != nullptr;
    uint32_t* s_pts = s_dyn + smask_words + wide_words;
    uint32_t* s_h8 = s_pts + (need_2z ? 2u * a.npts : 0u);
    if constexpr (RESTORE) load_sign_masks(s_smask, a.signs, a.cols, tid);
    if constexpr (LDS_PTS) {
        if (need_2z)
            for (uint32_t i = tid; i < 2u * a.npts; i += kBlock) s_pts[i] = a.pts[i];
        if constexpr (RESTORE)
            for (uint32_t i = tid; i < 2u * a.npts; i += kBlock) s_h8[i] = a.h8[i];
    }
    if constexpr (RESTORE || LDS_PTS) __syncthreads();
    const uint32_t* pts = LDS_PTS ? s_pts : a.pts;
    const LaneFwht lf = lane_fwht<(HB > 128 ? 128 : (HB < 8 ? 8 : HB))>(lane);
    const uint32_t lpos = wv * kWave + (lane & ~15u) + lf.logical;
    const uint32_t glast = a.groups - 1u;

    // The indices and row scales of the next tile are loaded while this tile is
    // decoded (the per-group work is short, so a prefetch within the tile
    // cannot cover the memory latency).
    const bool need_s = a.q != nullptr || RESTORE;
    uint32_t nidx[kItems];
    float ns[kItems];
    auto load_tile = [&](uint32_t tile) {
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const uint32_t gn = min(tile * kTileGroups + uint32_t(j) * kBlock + lpos, glast);
            nidx[j] = a.core_idx[gn];
            ns[j] = need_s ? a.scale[fdiv(gn, a.gpr_div)] : 0.0f;
        }
    };
    // The loads are unconditional (indices past the end read the last group):
    // a conditional prefetch merges old and new values at the branch and the
    // merge waits for the loads at once.
    load_tile(blockIdx.x);
    for (uint32_t tile = blockIdx.x; tile < a.num_tiles; tile += gridDim.x) {
        uint32_t cidx[kItems];
        float cs[kItems];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            cidx[j] = nidx[j];
            cs[j] = ns[j];
        }
        load_tile(tile + gridDim.x);
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const uint32_t g = tile * kTileGroups + uint32_t(j) * kBlock + lpos;
            const bool live = g < a.groups;
            const uint32_t gl = min(g, glast);
            const uint32_t idx = cidx[j];
            const uint32_t row = fdiv(gl, a.gpr_div);
            const float s_row = cs[j];
            uint32_t flags = 0;
            uint32_t t0 = 0x40404040u, t1 = 0x40404040u;   // 2z + 64 bytes (z = 0)
            bool big = false;
            int tb[8];
            uint32_t h0 = 0u, h1 = 0u;   // H_8 (2z) signed bytes (table restore)
            if (idx < a.npts) {
                if (!LDS_PTS || need_2z) {
                    t0 = pts[2u * idx];
                    t1 = pts[2u * idx + 1u];
                }
                if constexpr (RESTORE && LDS_PTS) {
                    h0 = s_h8[2u * idx];
                    h1 = s_h8[2u * idx + 1u];
                }
            } else if (idx == 0xFFFFu) {
                const uint32_t b = fdiv(gl, a.gpb_div);
                if (find_record(a.esc, a.offsets, b, gl - b * a.gpb, a.gpb, tb)) {
                    big = true;
                } else if (live) {
                    flags |= E8Q_STATUS_ESC_MISSING;
                }
            } else if (live) {
                flags |= E8Q_STATUS_BAD_INDEX;
            }
            const float s = s_row;
            const bool bad = !(s > 0.0f) || __builtin_isinf(s);
            if (live && a.two_z) {
                uint2 o;
                if (big) {
                    o = pack_i8x8(tb, flags);
                } else {
                    // bytes 2z + 64 in [58, 70] -> signed 2z bytes
                    const uint32_t x0 = t0 ^ 0x40404040u, x1 = t1 ^ 0x40404040u;
                    o = make_uint2(x0 | ((x0 & 0x40404040u) << 1), x1 | ((x1 & 0x40404040u) << 1));
                }
                *reinterpret_cast<uint2*>(a.two_z + uint64_t(g) * 8) = o;
            }
            if (live && a.q) {
                float q[8];
                if (!big && s > 0x1p-100f && s < 0x1p100f) {
                    const float sh = 0.5f * s, sm = -32.0f * s;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        q[i] = fmaf(float((t0 >> (8 * i)) & 0xFFu), sh, sm);
                        q[4 + i] = fmaf(float((t1 >> (8 * i)) & 0xFFu), sh, sm);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int ti = big ? tb[i] : int((((i < 4 ? t0 : t1) >> (8 * (i & 3))) & 0xFFu)) - 64;
                        q[i] = bad ? 0.0f : s * (float(ti) * 0.5f);
                    }
                }
                if (a.q_bf16) {
                    uint4 p;   // q is never NaN: the hardware conversion rounds to nearest even
                    p.x = bf16x2_rne_dec(q[0], q[1]);
                    p.y = bf16x2_rne_dec(q[2], q[3]);
                    p.z = bf16x2_rne_dec(q[4], q[5]);
                    p.w = bf16x2_rne_dec(q[6], q[7]);
                    // streamed out, never read back here: nontemporal
                    const u32x4 pv = {p.x, p.y, p.z, p.w};
                    __builtin_nontemporal_store(pv, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.q) + uint64_t(g) * 8));
                } else {
                    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.q) + uint64_t(g) * 8);
                    dst[0] = make_float4(q[0], q[1], q[2], q[3]);
                    dst[1] = make_float4(q[4], q[5], q[6], q[7]);
                }
            }
            if constexpr (RESTORE) {
                // inverse rotation across the block; every lane takes part
                float r[8];
                if constexpr (LDS_PTS) {
                    if (big) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) r[i] = float(tb[i]);
                        fwht_inlane<8>(r);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            r[i] = float(int32_t(h0 << (24 - 8 * i)) >> 24);
                            r[4 + i] = float(int32_t(h1 << (24 - 8 * i)) >> 24);
                        }
                    }
                } else {
                    float rcorr;
                    if (big) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) r[i] = float(tb[i]);
                        rcorr = 0.0f;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            r[i] = float((t0 >> (8 * i)) & 0xFFu);
                            r[4 + i] = float((t1 >> (8 * i)) & 0xFFu);
                        }
                        rcorr = 512.0f;
                    }
                    fwht_inlane<8>(r);
                    r[0] -= rcorr;
                }
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
                        p.x = bf16x2_rne_dec(y[0], y[1]) ^ m.x;
                        p.y = bf16x2_rne_dec(y[2], y[3]) ^ m.y;
                        p.z = bf16x2_rne_dec(y[4], y[5]) ^ m.z;
                        p.w = bf16x2_rne_dec(y[6], y[7]) ^ m.w;
                        // streamed out, never read back here: nontemporal
                        __builtin_nontemporal_store(p.x, reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.w_hat) + uint64_t(g) * 8));
                        __builtin_nontemporal_store(p.y, reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.w_hat) + uint64_t(g) * 8) + 1);
                        __builtin_nontemporal_store(p.z, reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.w_hat) + uint64_t(g) * 8) + 2);
                        __builtin_nontemporal_store(p.w, reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.w_hat) + uint64_t(g) * 8) + 3);
                    } else {
                        flip_f32(y, m);
                        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.w_hat) + uint64_t(g) * 8);
                        dst[0] = make_float4(y[0], y[1], y[2], y[3]);
                        dst[1] = make_float4(y[4], y[5], y[6], y[7]);
                    }
                }
            }
            if (live && (a.q || RESTORE) && bad) flags |= E8Q_STATUS_BAD_SCALE;
            flush_status(flags, a.status);
        }
    }
}

// The restore's blocks loop over 16 tiles each (at least one block per resident
// slot): more blocks than fit at once balance the CUs better than resident
// blocks, and 16 tiles amortize a block's table set-up.
template <typename K>
static void launch_restore(K kernel, const DecodeArgs& a, size_t lds, hipStream_t st) {
    const uint64_t resident = resident_grid(reinterpret_cast<const void*>(kernel), kBlock, lds, a.num_tiles);
    const uint64_t grid = std::min<uint64_t>(a.num_tiles, std::max<uint64_t>(resident, (uint64_t(a.num_tiles) + 15) / 16));
    launch(kernel, dim3(unsigned(grid)), dim3(kBlock), lds, st, a);
}

template <bool RESTORE, bool LDS_PTS>
static void launch_decode(int hb, const DecodeArgs& a, size_t lds, hipStream_t st) {
    if constexpr (!RESTORE) {
        // Without the restore the block size plays no part, and a block's set-up
        // is one copy of the point table: one block per tile (the hardware
        // dispatcher keeps every CU full) decodes faster than resident blocks
        // that loop over tiles.
        launch((decode_kernel<8, false, LDS_PTS>), dim3(a.num_tiles), dim3(kBlock), lds, st, a);
        return;
    }
    switch (hb) {
        case 8: launch_restore(decode_kernel<8, RESTORE, LDS_PTS>, a, lds, st); break;
        case 16: launch_restore(decode_kernel<16, RESTORE, LDS_PTS>, a, lds, st); break;
        case 32: launch_restore(decode_kernel<32, RESTORE, LDS_PTS>, a, lds, st); break;
        case 64: launch_restore(decode_kernel<64, RESTORE, LDS_PTS>, a, lds, st); break;
        case 128: launch_restore(decode_kernel<128, RESTORE, LDS_PTS>, a, lds, st); break;
        case 256: launch_restore(decode_kernel<256, RESTORE, LDS_PTS>, a, lds, st); break;
        case 512: launch_restore(decode_kernel<512, RESTORE, LDS_PTS>, a, lds, st); break;
        case 1024: launch_restore(decode_kernel<1024, RESTORE, LDS_PTS>, a, lds, st); break;
        case 2048: launch_restore(decode_kernel<2048, RESTORE, LDS_PTS>, a, lds, st); break;
        case 4096: launch_restore(decode_kernel<4096, RESTORE, LDS_PTS>, a, lds, st); break;
        default: break;
    }
}

static size_t decode_ws_bytes(int64_t batch) { return (size_t(batch + 1) * 8 + 255) & ~size_t(255); }

}  // namespace e8q

extern "C" size_t e8q_decode_workspace_size(int64_t batch) {
    if (batch <= 0 || batch >= (int64_t(1) << 32)) return 0;
    return e8q::decode_ws_bytes(batch);
}

extern "C" e8q_status_t e8q_decode_core_escape(const uint16_t* core_idx, const e8q_escape_t* esc,
                                               int64_t esc_capacity, const int64_t* esc_count,
                                               int64_t batch, int64_t rows, int64_t cols,
                                               int32_t core_bound, const float* row_scale,
                                               const int8_t* signs, int32_t had_block, int8_t* two_z_out,
                                               void* q_out, e8q_dtype_t q_dtype, void* w_hat_out,
                                               e8q_dtype_t w_hat_dtype, void* workspace,
                                               size_t workspace_bytes, uint32_t* status_dev, void* stream) {
    using namespace e8q;
    if (!core_idx || !esc_count || !status_dev || !workspace) return E8Q_ERR_INVALID;
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 8) return E8Q_ERR_INVALID;
    if (core_bound < 0 || core_bound > 40) return E8Q_ERR_INVALID;
    if (esc_capacity < 0 || (esc_capacity > 0 && !esc)) return E8Q_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(esc) & 3u) return E8Q_ERR_INVALID;   // records are read as 32-bit words
    if (!two_z_out && !q_out && !w_hat_out) return E8Q_ERR_INVALID;
    if ((q_out || w_hat_out) && !row_scale) return E8Q_ERR_INVALID;
    if (q_out && q_dtype != E8Q_F32 && q_dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    if (w_hat_out) {
        if (w_hat_dtype != E8Q_F32 && w_hat_dtype != E8Q_BF16) return E8Q_ERR_INVALID;
        const e8q_status_t st = check_block(signs, had_block, cols);
        if (st != E8Q_OK) return st;
    }
    if (batch >= (int64_t(1) << 32)) return E8Q_ERR_UNSUPPORTED;
    if (workspace_bytes < decode_ws_bytes(batch) || (reinterpret_cast<uintptr_t>(workspace) & 7u))
        return E8Q_ERR_INVALID;
    const double groups = double(batch) * double(rows) * double(cols / 8);
    if (groups >= 4294967295.0 || double(rows) * double(cols / 8) >= 4294967295.0) return E8Q_ERR_UNSUPPORTED;
    const bool restore = w_hat_out != nullptr;
    const size_t base_lds = restore ? size_t(cols / 2) * 4 + (had_block > 128 ? size_t(8 * kBlock) * 4 : 0) : 0;
    if (base_lds > 60 * 1024) return E8Q_ERR_UNSUPPORTED;

    e8q_status_t err = E8Q_OK;
    const DevTable* tab = get_table(core_bound, err);
    if (!tab) return err;

    DecodeArgs a;
    a.core_idx = core_idx;
    a.esc = reinterpret_cast<const uint32_t*>(esc);
    a.offsets = static_cast<const uint64_t*>(workspace);
    a.gpr = uint32_t(cols / 8);
    a.gpb = uint32_t(uint64_t(rows) * a.gpr);
    a.groups = uint32_t(uint64_t(batch) * a.gpb);
    a.gpr_div = make_fastdiv(a.gpr);
    a.gpb_div = make_fastdiv(a.gpb);
    a.scale = row_scale;
    a.kappa = kappa_for(had_block);
    a.signs = signs;
    a.cols = uint32_t(cols);
    a.pts = tab->dpoints;
    a.h8 = tab->dh8;
    a.npts = uint32_t(tab->size);
    a.two_z = two_z_out;
    a.q = q_out;
    a.q_bf16 = q_dtype == E8Q_BF16;
    a.w_hat = w_hat_out;
    a.w_hat_bf16 = w_hat_dtype == E8Q_BF16;
    a.status = status_dev;
    a.num_tiles = uint32_t((uint64_t(a.groups) + kTileGroups - 1) / kTileGroups);

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    launch(decode_offsets_kernel, dim3(1), dim3(1024), 0, s, esc_count, uint32_t(batch),
                       uint64_t(esc_capacity), static_cast<uint64_t*>(workspace));
    const bool need_2z = q_out != nullptr || two_z_out != nullptr;
    const size_t pts_lds = size_t(a.npts) * 8 * ((need_2z ? 1 : 0) + (restore ? 1 : 0));
    const bool lds_pts = base_lds + pts_lds <= 60 * 1024;
    const size_t lds = base_lds + (lds_pts ? pts_lds : 0);
    if (restore) {
        if (lds_pts) launch_decode<true, true>(had_block, a, lds, s);
        else launch_decode<true, false>(had_block, a, lds, s);
    } else {
        if (lds_pts) launch_decode<false, true>(0, a, lds, s);
        else launch_decode<false, false>(0, a, lds, s);
    }
    return launch_status();
}

// ---------------------------------------------------------------- GEMV
//
// e8q_gemv_core_escape: y = W_hat x straight from the exported form.  With
// W_hat = R^T (s z) and R orthogonal, y_r = s_r sum_g z_g . x~_g where
// x~ = R x = kappa_b H_b (sigma * x) is computed once per activation vector
// (rotate_act_kernel, the forward rotation on the projection's lanes), so the
// product never materializes W_hat: each row reads its 16-bit indices (2 bits
// per weight) and one table entry per group.  gemv_kernel keeps x~ of one
// batch item in LDS; a wave owns a row at a time, its lanes stride over the
// row's groups, and a cross-lane sum finishes the row.

namespace e8q {

struct GemvArgs {
    const uint16_t* core_idx;
    const uint32_t* esc;
    const uint64_t* offsets;
    const float* xt;            // [batch, m, cols] rotated activations
    const float* scale;
    const uint32_t* pts;
    uint32_t npts;
    uint32_t rows;
    uint32_t cols;
    uint32_t gpr;
    uint32_t rows_per_block;
    float* y;                   // [batch, m, rows]
    uint32_t* status;
};

constexpr int kGemvThreads = 512;
constexpr int kGemvRows = 128;

constexpr int kGemvR = 4;   // rows a wave works on at once (x~ is read once for all of them)

// Four signed 2z bytes of one word to floats.
__device__ __forceinline__ void unpack4s(uint32_t sb, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = float(int32_t(sb << (24 - 8 * i)) >> 24);
}

// 2z of a slot that is not a core index (escape record, or malformed).
__device__ __forceinline__ void special_point(const GemvArgs& a, uint32_t b, uint32_t gib, uint32_t idx, float* z,
                                           uint32_t& flags) {
    int tb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (idx != 0xFFFFu)
        flags |= E8Q_STATUS_BAD_INDEX;
    else if (!find_record(a.esc, a.offsets, b, gib, a.rows * a.gpr, tb))
        flags |= E8Q_STATUS_ESC_MISSING;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = float(tb[i]);
}

template <int M, bool LDS_PTS>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
    extern __shared__ uint32_t s_dyn[];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wv = tid >> 6;
    const uint32_t b = blockIdx.y;
    float* s_xt = reinterpret_cast<float*>(s_dyn);
    uint32_t* s_pts = s_dyn + M * a.cols;
    {
        const float4* src = reinterpret_cast<const float4*>(a.xt + uint64_t(b) * M * a.cols);
        float4* dst = reinterpret_cast<float4*>(s_xt);
        for (uint32_t i = tid; i < M * a.cols / 4u; i += kGemvThreads) dst[i] = src[i];
        if constexpr (LDS_PTS) {
            // table words as signed 2z bytes
            for (uint32_t i = tid; i < 2u * a.npts; i += kGemvThreads) {
                const uint32_t x = a.pts[i] ^ 0x40404040u;
                s_pts[i] = x | ((x & 0x40404040u) << 1);
            }
        }
    }
    __syncthreads();
    const uint32_t nlast = a.npts - 1u;
    const uint32_t r_begin = blockIdx.x * a.rows_per_block;
    const uint32_t r_end = min(r_begin + a.rows_per_block, a.rows);
    uint32_t flags = 0;
    for (uint32_t rw = r_begin + wv * kGemvR; rw < r_end; rw += (kGemvThreads / kWave) * kGemvR) {
        const uint32_t nr = min(uint32_t(kGemvR), r_end - rw);        // wave-uniform
        float acc[kGemvR][M];
#pragma unroll
        for (int r = 0; r < kGemvR; ++r)
#pragma unroll
            for (int t = 0; t < M; ++t) acc[r][t] = 0.0f;
        // rows past the end repeat the last row (computed, never written)
        const uint16_t* rowp[kGemvR];
#pragma unroll
        for (int r = 0; r < kGemvR; ++r)
            rowp[r] = a.core_idx + (uint64_t(b) * a.rows + rw + min(uint32_t(r), nr - 1u)) * a.gpr;
        uint32_t nxt[kGemvR];
#pragma unroll
        for (int r = 0; r < kGemvR; ++r) nxt[r] = lane < a.gpr ? uint32_t(rowp[r][lane]) : 0u;
        for (uint32_t g = lane; g < a.gpr; g += kWave) {
            uint32_t idx[kGemvR];
#pragma unroll
            for (int r = 0; r < kGemvR; ++r) {
                idx[r] = nxt[r];
                const uint32_t gn = g + kWave;
                nxt[r] = gn < a.gpr ? uint32_t(rowp[r][gn]) : 0u;
            }
            float xv[M][8];
#pragma unroll
            for (int t = 0; t < M; ++t) {
                const float4* xp = reinterpret_cast<const float4*>(s_xt + t * a.cols + g * 8u);
                const float4 x0 = xp[0], x1 = xp[1];
                xv[t][0] = x0.x; xv[t][1] = x0.y; xv[t][2] = x0.z; xv[t][3] = x0.w;
                xv[t][4] = x1.x; xv[t][5] = x1.y; xv[t][6] = x1.z; xv[t][7] = x1.w;
            }
#pragma unroll
            for (int r = 0; r < kGemvR; ++r) {
                const uint32_t ii = min(idx[r], nlast);
                float z[8];
                if constexpr (LDS_PTS) {
                    unpack4s(s_pts[2u * ii], z);
                    unpack4s(s_pts[2u * ii + 1u], z + 4);
                } else {
                    const uint32_t x0 = a.pts[2u * ii] ^ 0x40404040u, x1 = a.pts[2u * ii + 1u] ^ 0x40404040u;
                    unpack4s(x0 | ((x0 & 0x40404040u) << 1), z);
                    unpack4s(x1 | ((x1 & 0x40404040u) << 1), z + 4);
                }
                const bool special = idx[r] > nlast;
                if (__ballot(special)) {
                    if (special && uint32_t(r) < nr)
                        special_point(a, b, (rw + uint32_t(r)) * a.gpr + g, idx[r], z, flags);
                }
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    float s0 = z[0] * xv[t][0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) s0 = fmaf(z[i], xv[t][i], s0);
                    acc[r][t] += s0;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kGemvR; ++r)
#pragma unroll
            for (int t = 0; t < M; ++t)
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) acc[r][t] += __shfl_xor(acc[r][t], off, 64);
        if (lane < nr) {
            float sel[M];
#pragma unroll
            for (int t = 0; t < M; ++t) {
                sel[t] = acc[0][t];
#pragma unroll
                for (int r = 1; r < kGemvR; ++r) sel[t] = lane == uint32_t(r) ? acc[r][t] : sel[t];
            }
            const uint32_t r = rw + lane;
            const float s = a.scale[uint64_t(b) * a.rows + r];
            const bool bad = !(s > 0.0f) || __builtin_isinf(s);
            if (bad) flags |= E8Q_STATUS_BAD_SCALE;
#pragma unroll
            for (int t = 0; t < M; ++t) a.y[(uint64_t(b) * M + t) * a.rows + r] = bad ? 0.0f : (0.5f * s) * sel[t];
        }
    }
    flush_status(flags, a.status);
}

// ---------------------------------------------------------------------------
// The GEMV on the matrix cores (rows of a multiple of 32 groups, 16-byte
// aligned indices).  One 16x16x32 bf16 MFMA takes 16 rows x 4 groups:
//   A (16 x 32): the rows' points of the four groups, read from a table that
//     holds every core point's 2z as 8 bfloat16 (exact: |2z| <= 12); entry
//     npts is the zero point, taken by escaped and malformed slots;
//   B (32 x 16): the same groups' activations split as x~ = hi + mid + lo
//     (bfloat16, round to nearest even; |x~ - hi - mid - lo| <= 2^-24 |x~|),
//     column 3v + p holding part p of vector v, columns >= 3M zero;
//   D[i][3v + p] = the row's 32 products with part p, each product exact.
// Lane l holds row l % 16 of the tile in A and column l % 16 in B and D (D row
// 4 (l / 16) + r in element r).  A wave walks its 16 rows in chunks of 32
// groups: lane quarter q = l / 16 loads the 16-byte index word of groups
// 32c + 8q ... 32c + 8q + 7 (a whole 64-byte row segment per four lanes), and
// step s of the chunk puts group 32c + 8q + s in K slice q (the order of the
// groups along K is free).  Index words are loaded four chunks ahead, also
// across the wave's tiles, into four fixed registers.  Steps go in pairs: the
// first MFMA starts from 0, the second accumulates onto it (64 products in an
// order the hardware chooses); the pairs are added in float32 in order, 8
// pairs (512 columns) per partial sum, the partials in order.  Escaped and malformed slots read the table's
// zero entry; the sweep only counts the escaped ones (per tile, in the
// workspace) and flags the malformed ones, and gemv_escape_kernel then adds
// the escaped slots' records to the finished rows.
constexpr uint32_t kGmRows = 16;
constexpr int kGmAhead = 4;   // index words (chunks) loaded ahead

typedef __bf16 gm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gm_f32x4 __attribute__((ext_vector_type(4)));

struct GemvMfmaArgs {
    const uint16_t* core_idx;
    const uint32_t* esc;
    const int64_t* esc_count;
    uint64_t esc_capacity;
    const uint64_t* offsets;   // record offsets per item (decode_offsets_kernel), or null:
                               // each escape block then sums the counts before its item
    const float* xt;           // [batch, m, cols] x~ (float32), for the escaped slots
    const uint4* xb;           // [batch, m, 3, gpr] x~ parts hi, mid, lo (8 bf16 per group)
    uint32_t* tile_esc;        // [batch, tiles_per_b] escaped slots per 16-row tile
    const float* scale;
    const uint4* tab;          // [npts + 1] points as 8 bf16 (entry npts: zero)
    const uint32_t* pts8;      // [npts] points as 2z + 64 bytes, two words each (int8 kernel)
    uint32_t npts;
    uint32_t rows;
    uint32_t gpr;
    uint32_t tiles_per_b;      // ceil(rows / 16)
    uint32_t tiles;            // batch * tiles_per_b
    float* y;
    uint32_t* status;
};

// LDS accesses of one wave, ordered across its lanes.
__device__ __forceinline__ void gm_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work units: (batch item, kWaves consecutive tiles); each wave takes one
// tile of a unit, a block a contiguous range of units (so its waves read
// neighbouring rows).  This kernel serves the cores of 4096 points or more
// (B >= 24; smaller cores take gemv_i8_kernel): the point table and the
// activation parts are read from global memory.
template <int M>
__global__ __launch_bounds__(512, 4) void gemv_mfma_kernel(GemvMfmaArgs a) {
    constexpr uint32_t kWaves = 8u;
    extern __shared__ uint4 s_gm[];
    // the wave index in a scalar register: the index ring's bookkeeping is wave-uniform
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    float* s_red = reinterpret_cast<float*>(s_gm) + wv * 256u;
    const uint4* tab = a.tab;
    const uint32_t i16 = lane & 15u, q = lane >> 4;
    const uint32_t nc = a.gpr >> 5;                 // chunks of 32 groups per row
    const uint32_t ncp = (nc + uint32_t(kGmAhead) - 1u) / uint32_t(kGmAhead) * uint32_t(kGmAhead);
    const uint32_t vcol = i16 / 3u, pcol = i16 - 3u * vcol;
    const bool bcol = i16 < 3u * M;
    const gm_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t flags = 0;

    const uint32_t units_per_b = (a.tiles_per_b + kWaves - 1u) / kWaves;
    const uint32_t units = (a.tiles / a.tiles_per_b) * units_per_b;
    const uint32_t per = (units + gridDim.x - 1u) / gridDim.x;
    const uint32_t u_begin = min(blockIdx.x * per, units), u_end = min(u_begin + per, units);
    // this wave's tile of unit u (within its batch item), or tiles_per_b
    const auto wave_tile = [&](uint32_t u) { return (u % units_per_b) * kWaves + wv; };
    const auto row_words = [&](uint32_t u) {
        const uint32_t bb = u / units_per_b;
        const uint32_t rr = min(wave_tile(u) * kGmRows + i16, a.rows - 1u);
        return reinterpret_cast<const uint4*>(a.core_idx + (uint64_t(bb) * a.rows + rr) * a.gpr) + q;
    };
    // the index words run kGmAhead chunks ahead, on across this wave's tiles
    // (past its last tile the pipeline re-reads words it already has)
    uint32_t pf_u = u_begin, pf_c = 0;
    while (pf_u < u_end && wave_tile(pf_u) >= a.tiles_per_b) ++pf_u;
    const uint4* pf_ip = pf_u < u_end ? row_words(pf_u) : reinterpret_cast<const uint4*>(a.core_idx) + q;
    const auto next_word = [&]() {
        const uint4 w = pf_ip[4u * min(pf_c, nc - 1u)];   // padding chunks re-read the last word
        if (++pf_c == ncp) {
            pf_c = 0;
            if (pf_u < u_end) {
                do ++pf_u; while (pf_u < u_end && wave_tile(pf_u) >= a.tiles_per_b);
                if (pf_u < u_end) pf_ip = row_words(pf_u);
            }
        }
        return w;
    };
    uint4 wq[kGmAhead];
#pragma unroll
    for (int k = 0; k < kGmAhead; ++k) wq[k] = next_word();
    uint4 xc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) xc[s] = make_uint4(0u, 0u, 0u, 0u);
    for (uint32_t u = u_begin; u < u_end; ++u) {
        const uint32_t b = u / units_per_b;
        const uint32_t t = wave_tile(u);
        if (t >= a.tiles_per_b) continue;
        const uint32_t r0 = t * kGmRows;
        const bool row_ok = r0 + i16 < a.rows;
        const uint32_t row = row_ok ? r0 + i16 : a.rows - 1u;   // rows past the end repeat the last
        // this lane's activation part: step s of chunk c at xp[32c + s] ([batch, m, 3, gpr])
        const uint4* xp = a.xb + uint64_t(b) * M * 3u * a.gpr + (bcol ? i16 : 0u) * a.gpr + 8u * q;
        // the row scale of lane (row) l < 16, loaded now and used at the end
        const float s_row = a.scale[uint64_t(b) * a.rows + min(r0 + (lane & 15u), a.rows - 1u)];
        gm_f32x4 acc1 = zero, acc2 = zero;
        uint32_t nesc = 0;
        // One chunk: the word in its ring slot (loaded kGmAhead chunks ago),
        // whose refill is issued at once.  Every slot is a fixed register: the
        // loop body takes the slots in order, and a row's chunk count is padded
        // to a multiple of kGmAhead (padding chunks only refill), so no slot
        // rotates -- a rotation's register moves would wait for the newest load.
        const auto chunk = [&](uint4& slot, uint32_t c) {
            uint4 w = slot;
            slot = next_word();
            if (c < nc) {
                // only the 3M lanes of real columns load (the D columns of the
                // others are never read)
                if (bcol) {
#pragma unroll
                    for (int s = 0; s < 8; ++s)
                        xc[s] = xp[32u * c + uint32_t(s)];
                }
                // the largest of the eight 16-bit indices (packed 16-bit maxima)
                const gm_u16x2 mx = __builtin_elementwise_max(
                    __builtin_elementwise_max(__builtin_bit_cast(gm_u16x2, w.x), __builtin_bit_cast(gm_u16x2, w.y)),
                    __builtin_elementwise_max(__builtin_bit_cast(gm_u16x2, w.z), __builtin_bit_cast(gm_u16x2, w.w)));
                const bool big = uint32_t(mx.x > mx.y ? mx.x : mx.y) >= a.npts;
                if (__ballot(big)) {
                    // rare: escaped slots counted, malformed ones flagged, and
                    // every index past the table set to its zero entry
                    if (big) {
                        if (row_ok) {
#pragma unroll 1
                            for (uint32_t s = 0; s < 8; ++s) {
                                const uint32_t h = s >> 1;
                                const uint32_t word = h == 0 ? w.x : h == 1 ? w.y : h == 2 ? w.z : w.w;
                                const uint32_t id = (word >> (16u * (s & 1u))) & 0xFFFFu;
                                if (id == 0xFFFFu) ++nesc;
                                else if (id >= a.npts) flags |= E8Q_STATUS_BAD_INDEX;
                            }
                        }
                        const gm_u16x2 lim = {uint16_t(a.npts), uint16_t(a.npts)};
                        w.x = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.x), lim));
                        w.y = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.y), lim));
                        w.z = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.z), lim));
                        w.w = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.w), lim));
                    }
                }
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                // every index is now <= npts (entry npts: zero)
                const auto entry = [&](int s) { return tab[(wd[s >> 1] >> (16 * (s & 1))) & 0xFFFFu]; };
                const auto products = [&]() {
#pragma unroll
                    for (int s = 0; s < 8; s += 2) {
                        const uint4 p0 = entry(s);
                        const uint4 p1 = entry(s + 1);
                        const gm_f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(gm_bf16x8, p0), __builtin_bit_cast(gm_bf16x8, xc[s]), zero, 0, 0, 0);
                        const gm_f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(gm_bf16x8, p1), __builtin_bit_cast(gm_bf16x8, xc[s + 1]), d0, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc1[r] = acc1[r] + d[r];
                    }
                };
                products();
                if ((c & 1u) == 1u || c + 1u == nc) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc2[r] = acc2[r] + acc1[r];
                    acc1 = zero;
                }
            }
        };
        for (uint32_t c = 0; c < ncp; c += uint32_t(kGmAhead)) {
#pragma unroll
            for (int k = 0; k < kGmAhead; ++k) chunk(wq[k], c + uint32_t(k));
        }
        // D (16 rows x 16 columns); the tile's escaped slots
#pragma unroll
        for (int r = 0; r < 4; ++r) s_red[(4u * q + uint32_t(r)) * 16u + i16] = acc2[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) nesc += __shfl_xor(nesc, off, 64);
        if (lane == 0u) a.tile_esc[uint64_t(b) * a.tiles_per_b + t] = nesc;
        gm_wave_sync();
        if (lane < kGmRows && r0 + lane < a.rows) {
            const uint32_t r = r0 + lane;
            const float s = s_row;
            const bool bad = !(s > 0.0f) || __builtin_isinf(s);
            if (bad) flags |= E8Q_STATUS_BAD_SCALE;
            const float* d = s_red + lane * 16u;
#pragma unroll
            for (int v = 0; v < M; ++v) {
                const float dv = (d[3 * v] + d[3 * v + 1]) + d[3 * v + 2];
                a.y[(uint64_t(b) * M + uint32_t(v)) * a.rows + r] = bad ? 0.0f : (0.5f * s) * dv;
            }
        }
        gm_wave_sync();
    }
    flush_status(flags, a.status);
}

// ---------------------------------------------------------------------------
// The GEMV on the int8 matrix cores (same shapes as gemv_mfma_kernel, table and
// activations in LDS).  Each activation vector is held in fixed point: with e
// the exponent of its largest |x~| (2^(e-1) <= max < 2^e), N_k = rint(x~_k
// 2^(30-e)) (|N_k| <= 2^30) is written as four signed base-256 digits,
// N = ((D0 256 + D1) 256 + D2) 256 + D3, D_i in [-128, 127].  One
// v_mfma_i32_16x16x64_i8 takes 16 rows x 8 groups:
//   A (16 x 64): the rows' points as signed bytes 2z (8 bytes per table entry,
//     entry npts zero), two groups per lane;
//   B (64 x 16): the same groups' digits, column 4v + d holding digit d of
//     vector v (columns >= 4M unused);
//   D (16 x 16) int32, accumulated over the whole row: every product and sum
//     is exact (|2z_i| <= 6, |D| <= 128, cols < 2^19).
// The row's y is then (s/2) 2^(e-30) ((I0 256 + I1) 256 + I2) 256 + I3 from the
// four column sums (an exact int64, exact in float64 below 2^53), rounded once
// to float32 after one float64 product: the only errors are the fixed-point
// step (|x~ - N 2^(e-30)| <= 2^(e-31)) and those two roundings.  Lane l holds
// row l % 16 of the tile in A; lane quarter q = l / 16 loads the index word of
// groups 32c + 8q ... 32c + 8q + 7, and step s of the chunk puts groups
// 32c + 8q + 2s, +1 in its K slice.  The same byte positions of A and B hold
// the same group, so the K order the hardware uses does not matter.  Index
// words run kI8Ahead chunks ahead, as in gemv_mfma_kernel; escaped and
// malformed slots read the zero entry and are handled the same way.  A vector
// with a non-finite x~ gives NaN rows and E8Q_STATUS_NONFINITE.
typedef int gm_i32x4 __attribute__((ext_vector_type(4)));
constexpr int kI8Ahead = 4;   // index words (chunks) loaded ahead
constexpr uint32_t kI8TabEntries = 4096;   // table entries in LDS (cores below 4096 points + the zero entry)

template <int M>
__global__ __launch_bounds__(1024, 4) void gemv_i8_kernel(GemvMfmaArgs a) {
    constexpr uint32_t kWaves = 16u;
    constexpr uint32_t kThreads = kWaves * kWave;
    constexpr uint32_t NCOL = 4u * uint32_t(M);
    // the table at a fixed LDS address (its offsets fold into the reads), then
    // the dynamic LDS: digits and the row exchange
    __shared__ uint2 s_tab[kI8TabEntries];
    extern __shared__ uint4 s_gm[];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t cols = a.gpr * 8u;
    const uint32_t xs_n = NCOL * (a.gpr / 2u);        // 16-byte digit entries: per pair of groups, per column
    uint4* s_x = s_gm;
    int* s_red = reinterpret_cast<int*>(s_gm + xs_n) + wv * 256u;
    // while a batch item's digits are staged the exchange area holds the
    // per-wave maxima and the exponents
    uint32_t (*s_mx)[M] = reinterpret_cast<uint32_t (*)[M]>(s_gm + xs_n);
    int* s_e = reinterpret_cast<int*>(s_gm + xs_n) + kWaves * M;
    // points as signed bytes: (b - 64) mod 256 per byte of b = 2z + 64, no borrow across bytes
    for (uint32_t i = tid; i <= a.npts; i += kThreads) {
        uint32_t p0 = 0x40404040u, p1 = 0x40404040u;
        if (i < a.npts) {
            p0 = a.pts8[2u * i];
            p1 = a.pts8[2u * i + 1u];
        }
        s_tab[i] = make_uint2(((p0 | 0x80808080u) - 0x40404040u) ^ 0x80808080u,
                              ((p1 | 0x80808080u) - 0x40404040u) ^ 0x80808080u);
    }
    __syncthreads();
    const uint32_t i16 = lane & 15u, q = lane >> 4;
    const uint32_t nc = a.gpr >> 5;
    const uint32_t ncp = (nc + uint32_t(kI8Ahead) - 1u) / uint32_t(kI8Ahead) * uint32_t(kI8Ahead);
    const bool bcol = i16 < NCOL;
    uint32_t flags = 0;

    const uint32_t units_per_b = (a.tiles_per_b + kWaves - 1u) / kWaves;
    const uint32_t units = (a.tiles / a.tiles_per_b) * units_per_b;
    const uint32_t per = (units + gridDim.x - 1u) / gridDim.x;
    const uint32_t u_begin = min(blockIdx.x * per, units), u_end = min(u_begin + per, units);
    const auto wave_tile = [&](uint32_t u) { return (u % units_per_b) * kWaves + wv; };
    const auto row_words = [&](uint32_t u) {
        const uint32_t bb = u / units_per_b;
        const uint32_t rr = min(wave_tile(u) * kGmRows + i16, a.rows - 1u);
        return reinterpret_cast<const uint4*>(a.core_idx + (uint64_t(bb) * a.rows + rr) * a.gpr) + q;
    };
    uint32_t pf_u = u_begin, pf_c = 0;
    while (pf_u < u_end && wave_tile(pf_u) >= a.tiles_per_b) ++pf_u;
    const uint4* pf_ip = pf_u < u_end ? row_words(pf_u) : reinterpret_cast<const uint4*>(a.core_idx) + q;
    const auto next_word = [&]() {
        const uint4 w = pf_ip[4u * min(pf_c, nc - 1u)];
        if (++pf_c == ncp) {
            pf_c = 0;
            if (pf_u < u_end) {
                do ++pf_u; while (pf_u < u_end && wave_tile(pf_u) >= a.tiles_per_b);
                if (pf_u < u_end) pf_ip = row_words(pf_u);
            }
        }
        return w;
    };
    uint4 wq[kI8Ahead];
#pragma unroll
    for (int k = 0; k < kI8Ahead; ++k) wq[k] = next_word();
    uint32_t staged = 0xFFFFFFFFu;
    int ev[M];
#pragma unroll
    for (int v = 0; v < M; ++v) ev[v] = 0;
    for (uint32_t u = u_begin; u < u_end; ++u) {
        const uint32_t b = u / units_per_b;
        if (b != staged) {   // block-uniform
            __syncthreads();
            const float* xv = a.xt + uint64_t(b) * M * cols;
            // largest |x~| bits per vector (NaN and infinity above every finite value)
            uint32_t mx[M];
#pragma unroll
            for (int v = 0; v < M; ++v) {
                mx[v] = 0u;
                for (uint32_t i = tid; i < cols; i += kThreads)
                    mx[v] = max(mx[v], __float_as_uint(xv[uint64_t(v) * cols + i]) & 0x7FFFFFFFu);
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mx[v] = max(mx[v], uint32_t(__shfl_xor(mx[v], off, 64)));
                if (lane == 0u) s_mx[wv][v] = mx[v];
            }
            __syncthreads();
            if (tid < uint32_t(M)) {
                uint32_t m = 0u;
                for (uint32_t k = 0; k < kWaves; ++k) m = max(m, s_mx[k][tid]);
                // e with 2^(e-1) <= max < 2^e; 0 for an all-zero vector; 255 marks a non-finite one
                s_e[tid] = m >= 0x7F800000u ? 255 : (m == 0u ? 0 : __builtin_amdgcn_frexp_expf(__uint_as_float(m)));
            }
            __syncthreads();
#pragma unroll
            for (int v = 0; v < M; ++v) ev[v] = s_e[v];
            // digits in step order: entry ((4c + s) 4 + q) NCOL + n holds column n's
            // digits for groups 32c + 8q + 2s, +1, so that the lanes of one step
            // read consecutive entries
            for (uint32_t i = tid; i < uint32_t(M) * (a.gpr / 2u); i += kThreads) {
                const uint32_t v = i / (a.gpr / 2u), pr = i - v * (a.gpr / 2u);
                const uint32_t c = pr >> 4, qq = (pr >> 2) & 3u, st = pr & 3u;
                const float* src = xv + uint64_t(v) * cols + 16u * pr;
                int evv = ev[0];
#pragma unroll
                for (int w2 = 1; w2 < M; ++w2)
                    if (v == uint32_t(w2)) evv = ev[w2];
                const bool fin = evv != 255;   // digits of a non-finite vector are never used
                const int shv = fin ? 30 - evv : 0;
                uint32_t dg[4][4];
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int k = 0; k < 4; ++k) dg[d][k] = 0u;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const float xs = __builtin_ldexpf(src[k], shv);
                    int n = fin ? int(__builtin_rintf(xs)) : 0;   // |xs| <= 2^30
                    const int d3 = int(int8_t(uint8_t(n)));
                    n = (n - d3) >> 8;
                    const int d2 = int(int8_t(uint8_t(n)));
                    n = (n - d2) >> 8;
                    const int d1 = int(int8_t(uint8_t(n)));
                    const int d0 = (n - d1) >> 8;
                    const uint32_t sb = 8u * uint32_t(k & 3);
                    dg[0][k >> 2] |= (uint32_t(d0) & 0xFFu) << sb;
                    dg[1][k >> 2] |= (uint32_t(d1) & 0xFFu) << sb;
                    dg[2][k >> 2] |= (uint32_t(d2) & 0xFFu) << sb;
                    dg[3][k >> 2] |= (uint32_t(d3) & 0xFFu) << sb;
                }
                const uint32_t base = ((4u * c + st) * 4u + qq) * NCOL + 4u * v;
#pragma unroll
                for (int d = 0; d < 4; ++d) s_x[base + uint32_t(d)] = make_uint4(dg[d][0], dg[d][1], dg[d][2], dg[d][3]);
            }
            __syncthreads();
            staged = b;
        }
        const uint32_t t = wave_tile(u);
        if (t >= a.tiles_per_b) continue;
        const uint32_t r0 = t * kGmRows;
        const bool row_ok = r0 + i16 < a.rows;
        // lanes of unused columns read column 0's entry (an LDS broadcast; their D
        // columns are never read)
        const uint4* xp = s_x + (q * NCOL + (bcol ? i16 : 0u));
        const float s_row = a.scale[uint64_t(b) * a.rows + min(r0 + (lane & 15u), a.rows - 1u)];
        gm_i32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
        uint32_t nesc = 0;
        const auto chunk = [&](uint4& slot, uint32_t c) {
            uint4 w = slot;
            slot = next_word();
            if (c < nc) {
                const gm_u16x2 mxi = __builtin_elementwise_max(
                    __builtin_elementwise_max(__builtin_bit_cast(gm_u16x2, w.x), __builtin_bit_cast(gm_u16x2, w.y)),
                    __builtin_elementwise_max(__builtin_bit_cast(gm_u16x2, w.z), __builtin_bit_cast(gm_u16x2, w.w)));
                const bool big = uint32_t(mxi.x > mxi.y ? mxi.x : mxi.y) >= a.npts;
                if (__ballot(big)) {
                    if (big) {
                        if (row_ok) {
#pragma unroll 1
                            for (uint32_t s = 0; s < 8; ++s) {
                                const uint32_t h = s >> 1;
                                const uint32_t word = h == 0 ? w.x : h == 1 ? w.y : h == 2 ? w.z : w.w;
                                const uint32_t id = (word >> (16u * (s & 1u))) & 0xFFFFu;
                                if (id == 0xFFFFu) ++nesc;
                                else if (id >= a.npts) flags |= E8Q_STATUS_BAD_INDEX;
                            }
                        }
                        const gm_u16x2 lim = {uint16_t(a.npts), uint16_t(a.npts)};
                        w.x = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.x), lim));
                        w.y = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.y), lim));
                        w.z = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.z), lim));
                        w.w = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(gm_u16x2, w.w), lim));
                    }
                }
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                // the chunk's eight table reads and four digit reads first, then its
                // four MFMAs (entries are 8 bytes and every index is now <= npts < 4096)
                uint2 p0[4], p1[4];
                uint4 xc[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    p0[s] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(s_tab) +
                                                            ((wd[s] << 3) & 0x7FFF8u));
                    p1[s] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(s_tab) + (wd[s] >> 13));
                    xc[s] = xp[(4u * c + uint32_t(s)) * 4u * NCOL];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const gm_i32x4 av = {int(p0[s].x), int(p0[s].y), int(p1[s].x), int(p1[s].y)};
                    const gm_i32x4 bv = {int(xc[s].x), int(xc[s].y), int(xc[s].z), int(xc[s].w)};
                    if (s & 1) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc1, 0, 0, 0);
                    else acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc0, 0, 0, 0);
                }
            }
        };
        for (uint32_t c = 0; c < ncp; c += uint32_t(kI8Ahead)) {
#pragma unroll
            for (int k = 0; k < kI8Ahead; ++k) chunk(wq[k], c + uint32_t(k));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s_red[(4u * q + uint32_t(r)) * 16u + i16] = acc0[r] + acc1[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) nesc += __shfl_xor(nesc, off, 64);
        if (lane == 0u) a.tile_esc[uint64_t(b) * a.tiles_per_b + t] = nesc;
        gm_wave_sync();
        if (lane < kGmRows && r0 + lane < a.rows) {
            const uint32_t r = r0 + lane;
            const float s = s_row;
            const bool bad = !(s > 0.0f) || __builtin_isinf(s);
            if (bad) flags |= E8Q_STATUS_BAD_SCALE;
            const int* d = s_red + lane * 16u;
#pragma unroll
            for (int v = 0; v < M; ++v) {
                const int64_t yi = ((int64_t(d[4 * v]) * 256 + d[4 * v + 1]) * 256 + d[4 * v + 2]) * 256 + d[4 * v + 3];
                float yv;
                if (ev[v] == 255) {
                    yv = __uint_as_float(0x7FC00000u);
                    flags |= E8Q_STATUS_NONFINITE;
                } else {
                    yv = float((0.5 * double(s)) * __builtin_ldexp(double(yi), ev[v] - 30));
                }
                a.y[(uint64_t(b) * M + uint32_t(v)) * a.rows + r] = bad ? 0.0f : yv;
            }
        }
        gm_wave_sync();
    }
    flush_status(flags, a.status);
}

// The escaped slots of one batch item (one block each), after the sweep:
// the item's records are esc[first, end) with first / end the clipped
// running sums of the counts (as e8q_decode_core_escape's offsets).  The
// thread holding a row's first record adds 2z . x~ of every record of that
// row whose slot holds 0xFFFF and whose key differs from the previous
// record's, in order, in blocks of 32 (each block summed from 0, the block
// sums added in order), and adds (s / 2) times the sum to the row's y (not
// for rows with a bad scale, whose y stays 0).  An item whose escaped slots
// (counted by the sweep) outnumber those records lacks a record.
template <int M>
__global__ __launch_bounds__(1024) void gemv_escape_kernel(GemvMfmaArgs a) {
    __shared__ uint64_t s_sum[32];
    const uint32_t b = blockIdx.x, tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
    const uint32_t nw = blockDim.x >> 6;
    // records before this item, and this item's escaped slots
    uint64_t before = 0, slots = 0;
    if (!a.offsets)
        for (uint32_t i = tid; i < b; i += blockDim.x) before += a.esc_count[i] > 0 ? uint64_t(a.esc_count[i]) : 0ull;
    for (uint32_t i = tid; i < a.tiles_per_b; i += blockDim.x) slots += a.tile_esc[uint64_t(b) * a.tiles_per_b + i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        before += __shfl_xor(before, off, 64);
        slots += __shfl_xor(slots, off, 64);
    }
    if (lane == 0u) {
        s_sum[wv] = before;
        s_sum[16u + wv] = slots;
    }
    __syncthreads();
    before = 0;
    slots = 0;
    for (uint32_t w = 0; w < nw; ++w) {
        before += s_sum[w];
        slots += s_sum[16u + w];
    }
    const uint64_t own = a.esc_count[b] > 0 ? uint64_t(a.esc_count[b]) : 0ull;
    const uint64_t first = a.offsets ? a.offsets[b] : min(before, a.esc_capacity);
    const uint64_t end = a.offsets ? a.offsets[b + 1] : min(before + own, a.esc_capacity);
    const uint64_t gpb = uint64_t(a.rows) * a.gpr;
    const uint16_t* slot_idx = a.core_idx + uint64_t(b) * gpb;
    uint64_t matched = 0;
    for (uint64_t i = first + tid; i < end; i += blockDim.x) {
        const uint32_t key = a.esc[i * 5];
        const uint32_t pk = i > first ? a.esc[(i - 1) * 5] : 0xFFFFFFFFu;
        if (key >= gpb) continue;
        const uint32_t row = key / a.gpr;
        if (pk < gpb && pk / a.gpr == row) continue;   // not the row's first record
        float total[M], blk[M];
#pragma unroll
        for (int v = 0; v < M; ++v) total[v] = blk[v] = 0.0f;
        uint32_t in_blk = 0, prev = 0xFFFFFFFFu;
        for (uint64_t j = i; j < end; ++j) {
            const uint32_t kj = a.esc[j * 5];
            if (kj >= gpb || kj / a.gpr != row) break;
            if (kj != prev && slot_idx[kj] == 0xFFFFu) {
                const uint32_t* rec = a.esc + j * 5 + 1;
                float z[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t wd = rec[k];
                    z[2 * k] = float(int32_t(int16_t(uint16_t(wd & 0xFFFFu))));
                    z[2 * k + 1] = float(int32_t(int16_t(uint16_t(wd >> 16))));
                }
                const uint32_t g = kj - row * a.gpr;
#pragma unroll
                for (int v = 0; v < M; ++v) {
                    const float* x = a.xt + ((uint64_t(b) * M + uint32_t(v)) * a.gpr + g) * 8u;
                    float cs = z[0] * x[0];
#pragma unroll
                    for (int k = 1; k < 8; ++k) cs = fmaf(z[k], x[k], cs);
                    blk[v] += cs;
                }
                ++matched;
                if (++in_blk == 32u) {
#pragma unroll
                    for (int v = 0; v < M; ++v) {
                        total[v] += blk[v];
                        blk[v] = 0.0f;
                    }
                    in_blk = 0;
                }
            }
            prev = kj;
        }
        const float s = a.scale[uint64_t(b) * a.rows + row];
        if (s > 0.0f && !__builtin_isinf(s)) {
#pragma unroll
            for (int v = 0; v < M; ++v) {
                float* yp = a.y + (uint64_t(b) * M + uint32_t(v)) * a.rows + row;
                *yp = *yp + (0.5f * s) * (total[v] + blk[v]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) matched += __shfl_xor(matched, off, 64);
    __syncthreads();
    if (lane == 0u) s_sum[wv] = matched;
    __syncthreads();
    if (tid == 0u) {
        uint64_t m = 0;
        for (uint32_t w = 0; w < nw; ++w) m += s_sum[w];
        if (m != slots) atomicOr(a.status, uint32_t(E8Q_STATUS_ESC_MISSING));
    }
}

static size_t gemv_xt_bytes(int64_t batch, int64_t m, int64_t cols) {
    return (size_t(batch) * size_t(m) * size_t(cols) * 4 + 255) & ~size_t(255);
}

static size_t gemv_xb_bytes(int64_t batch, int64_t m, int64_t cols) {
    return (size_t(batch) * size_t(m) * size_t(cols / 8) * 48 + 255) & ~size_t(255);
}

// offsets, x~ (float32), x~ parts (3 x 8 bf16 per group), escaped slots per 16-row tile
static size_t gemv_ws_bytes(int64_t batch, int64_t m, int64_t rows, int64_t cols) {
    return decode_ws_bytes(batch) + gemv_xt_bytes(batch, m, cols) + gemv_xb_bytes(batch, m, cols) +
           ((size_t(batch) * size_t((rows + kGmRows - 1) / kGmRows) * 4 + 255) & ~size_t(255));
}

template <int M>
static void launch_gemv(bool lds_pts, const GemvArgs& a, dim3 grid, size_t lds, hipStream_t st) {
    if (lds_pts)
        launch((gemv_kernel<M, true>), grid, dim3(kGemvThreads), lds, st, a);
    else
        launch((gemv_kernel<M, false>), grid, dim3(kGemvThreads), lds, st, a);
}

// Dynamic LDS bytes of gemv_i8_kernel: the activation digits (4 bytes per
// element and vector) and the row exchange of 16 waves (the table's 32 KiB
// are static).
static size_t gemv_i8_lds(int64_t m, int64_t cols) {
    return size_t(m) * 4 * size_t(cols) + 16 * 256 * 4;
}

// Whether the matrix-core GEMV of these shapes runs on the int8 kernel: table
// in LDS (fewer than 4096 points: byte offsets from two shifts), digits in
// LDS, exact int32 row sums (cols < 2^19).
static bool gemv_use_i8(uint32_t npts, int64_t m, uint32_t gpr) {
    return npts < kI8TabEntries && gpr < (1u << 16) &&
           kI8TabEntries * 8 + gemv_i8_lds(m, int64_t(gpr) * 8) <= 160 * 1024;
}

template <int M>
static void launch_gemv_mfma(const GemvMfmaArgs& a, hipStream_t st) {
    const uint64_t batch = a.tiles / a.tiles_per_b;
    if (gemv_use_i8(a.npts, M, a.gpr)) {
        const uint64_t units = batch * ((a.tiles_per_b + 15) / 16);
        launch_tiles(gemv_i8_kernel<M>, a, units, 1024, gemv_i8_lds(M, int64_t(a.gpr) * 8), st);
        return;
    }
    // the bfloat16 kernel (cores of 4096 points or more): table and activation
    // parts from global memory
    const uint64_t units = batch * ((a.tiles_per_b + 7) / 8);
    launch_tiles(gemv_mfma_kernel<M>, a, units, 512, size_t(8 * 256 * 4), st);
}

}  // namespace e8q

extern "C" size_t e8q_gemv_workspace_size(int64_t batch, int64_t m, int64_t rows, int64_t cols) {
    if (batch <= 0 || batch >= (int64_t(1) << 32) || m <= 0 || rows <= 0 || rows >= (int64_t(1) << 32) || cols <= 0)
        return 0;
    return e8q::gemv_ws_bytes(batch, m, rows, cols);
}

extern "C" e8q_status_t e8q_gemv_core_escape(const uint16_t* core_idx, const e8q_escape_t* esc,
                                             int64_t esc_capacity, const int64_t* esc_count, int64_t batch,
                                             int64_t rows, int64_t cols, int32_t core_bound,
                                             const float* row_scale, const int8_t* signs, int32_t had_block,
                                             const void* x, e8q_dtype_t x_dtype, int64_t m, float* y_out,
                                             void* workspace, size_t workspace_bytes, uint32_t* status_dev,
                                             void* stream) {
    using namespace e8q;
    if (!core_idx || !esc_count || !row_scale || !x || !y_out || !status_dev || !workspace) return E8Q_ERR_INVALID;
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 8) return E8Q_ERR_INVALID;
    if (core_bound < 0 || core_bound > 40) return E8Q_ERR_INVALID;
    if (esc_capacity < 0 || (esc_capacity > 0 && !esc)) return E8Q_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(esc) & 3u) return E8Q_ERR_INVALID;
    if (x_dtype != E8Q_F32 && x_dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    if (m != 1 && m != 2 && m != 4) return E8Q_ERR_UNSUPPORTED;
    if (signs) {
        const e8q_status_t st = check_block(signs, had_block, cols);
        if (st != E8Q_OK) return st;
    }
    if (batch > 65535) return E8Q_ERR_UNSUPPORTED;   // one grid row per batch item
    if (workspace_bytes < gemv_ws_bytes(batch, m, rows, cols) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return E8Q_ERR_INVALID;
    const double groups = double(batch) * double(rows) * double(cols / 8);
    if (groups >= 4294967295.0 || double(batch) * double(m) * double(cols / 8) >= 4294967295.0 ||
        double(rows) * double(cols / 8) >= 4294967295.0)
        return E8Q_ERR_UNSUPPORTED;
    const size_t xt_lds = size_t(m) * size_t(cols) * 4;
    if (xt_lds > 96 * 1024) return E8Q_ERR_UNSUPPORTED;
    const int hb = signs ? had_block : 0;
    const size_t rot_lds = (hb > 0 ? size_t(cols / 2) * 4 : 0) + (hb > 128 ? size_t(8 * kBlock) * 4 : 0);
    if (rot_lds > 60 * 1024) return E8Q_ERR_UNSUPPORTED;

    e8q_status_t err = E8Q_OK;
    const DevTable* tab = get_table(core_bound, err);
    if (!tab) return err;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint64_t* offsets = static_cast<uint64_t*>(workspace);
    float* xt = reinterpret_cast<float*>(static_cast<char*>(workspace) + decode_ws_bytes(batch));
    uint4* xb = reinterpret_cast<uint4*>(reinterpret_cast<char*>(xt) + gemv_xt_bytes(batch, m, cols));
    uint32_t* tile_esc = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(xb) + gemv_xb_bytes(batch, m, cols));
    const uint32_t gpr = uint32_t(cols / 8);
    const uint64_t tiles = uint64_t(batch) * uint64_t((rows + kGmRows - 1) / kGmRows);
    const bool mfma = gpr % 32 == 0 && (reinterpret_cast<uintptr_t>(core_idx) & 15u) == 0 && tiles < (uint64_t(1) << 32);
    // the vector kernel finds escape records through the offsets; so do the
    // escape blocks of the matrix-core path when the batch is large (each
    // would otherwise sum the counts of every item before its own)
    const bool scan = !mfma || batch > 1024;
    if (scan)
        launch(decode_offsets_kernel, dim3(1), dim3(1024), 0, s, esc_count, uint32_t(batch),
               uint64_t(esc_capacity), offsets);

    RotArgs ra;
    ra.x = x;
    ra.xt = xt;
    // the bfloat16 parts only for the bfloat16 matrix-core kernel (the int8
    // kernel makes its digits from x~ itself)
    ra.xb = mfma && !gemv_use_i8(uint32_t(tab->size), m, uint32_t(cols / 8)) ? xb : nullptr;
    ra.signs = signs;
    ra.kappa = kappa_for(hb);
    ra.cols = uint32_t(cols);
    ra.gpr = uint32_t(cols / 8);
    ra.groups = uint32_t(uint64_t(batch) * uint64_t(m) * ra.gpr);
    ra.gpr_div = make_fastdiv(ra.gpr);
    ra.num_tiles = uint32_t((uint64_t(ra.groups) + kTileGroups - 1) / kTileGroups);
    if (x_dtype == E8Q_BF16)
        launch_rotate<uint16_t>(hb, ra, rot_lds, s);
    else
        launch_rotate<float>(hb, ra, rot_lds, s);

    if (mfma) {
        // the matrix-core path, then the escaped slots
        GemvMfmaArgs gm;
        gm.core_idx = core_idx;
        gm.esc = reinterpret_cast<const uint32_t*>(esc);
        gm.esc_count = esc_count;
        gm.esc_capacity = uint64_t(esc_capacity);
        gm.offsets = scan ? offsets : nullptr;
        gm.xt = xt;
        gm.xb = xb;
        gm.tile_esc = tile_esc;
        gm.scale = row_scale;
        gm.tab = tab->dpts_bf16;
        gm.pts8 = tab->dpoints;
        gm.npts = uint32_t(tab->size);
        gm.rows = uint32_t(rows);
        gm.gpr = gpr;
        gm.tiles_per_b = uint32_t((rows + kGmRows - 1) / kGmRows);
        gm.tiles = uint32_t(tiles);
        gm.y = y_out;
        gm.status = status_dev;
        if (m == 1) launch_gemv_mfma<1>(gm, s);
        else if (m == 2) launch_gemv_mfma<2>(gm, s);
        else launch_gemv_mfma<4>(gm, s);
        if (m == 1) launch(gemv_escape_kernel<1>, dim3(unsigned(batch)), dim3(1024), 0, s, gm);
        else if (m == 2) launch(gemv_escape_kernel<2>, dim3(unsigned(batch)), dim3(1024), 0, s, gm);
        else launch(gemv_escape_kernel<4>, dim3(unsigned(batch)), dim3(1024), 0, s, gm);
        return launch_status();
    }

    GemvArgs ga;
    ga.core_idx = core_idx;
    ga.esc = reinterpret_cast<const uint32_t*>(esc);
    ga.offsets = offsets;
    ga.xt = xt;
    ga.scale = row_scale;
    ga.pts = tab->dpoints;
    ga.npts = uint32_t(tab->size);
    ga.rows = uint32_t(rows);
    ga.cols = uint32_t(cols);
    ga.gpr = uint32_t(cols / 8);
    ga.rows_per_block = kGemvRows;
    ga.y = y_out;
    ga.status = status_dev;
    const size_t pts_lds = size_t(ga.npts) * 8;
    const bool lds_pts = xt_lds + pts_lds <= 64 * 1024;
    const size_t lds = xt_lds + (lds_pts ? pts_lds : 0);
    const dim3 grid(unsigned((rows + kGemvRows - 1) / kGemvRows), unsigned(batch));
    if (m == 1) launch_gemv<1>(lds_pts, ga, grid, lds, s);
    else if (m == 2) launch_gemv<2>(lds_pts, ga, grid, lds, s);
    else launch_gemv<4>(lds_pts, ga, grid, lds, s);
    return launch_status();
}
