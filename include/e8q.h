/*
 * e8q.h -- C ABI of the MI355X (gfx950) E8 lattice projection library.
 *
 * What it computes.  E8-QAT ("E8-QAT: Efficient 2-Bit Quantization-Aware
 * Training with Implicit Lattice Codebooks") quantizes LLM weights in groups
 * of eight: each group of normalized coordinates is sent by arithmetic alone
 * to its nearest point of the E8 lattice (no stored codebook is searched), an
 * identity straight-through estimator carries gradients back to the latent
 * weights, and for export every point is stored as a 16-bit index into a
 * finite core or, outside the core, as an exact sparse escape record
 * (abstract; captions of Figures 1(c), 2(a)-(c) and 6(c); Tables 3, 9, 10).
 * The pages leave the Hadamard transform and the scales out of their figure
 * (Figure 2 caption); the readings used here are stated with each call.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to memory the caller owns (for
 *     example torch tensors).  Work is enqueued on `stream` (a hipStream_t
 *     passed as void*; NULL = the legacy default stream) and runs
 *     asynchronously; nothing is synchronized before return.
 *   - The return value reports only host-side checks and the launch:
 *       E8Q_OK, E8Q_ERR_INVALID (a bad argument: null required pointer,
 *       non-positive size, cols not a multiple of 8, bad block size or core
 *       bound, too small workspace), E8Q_ERR_UNSUPPORTED (a dtype or size
 *       combination the library does not implement), E8Q_ERR_LAUNCH (the HIP
 *       launch failed), E8Q_ERR_DEVICE (a device query failed).  Nothing is
 *       launched when a check fails; E8Q_ERR_LAUNCH comes from this call's own
 *       launches, never from an error left by other code.
 *   - Conditions that depend on the data are reported by OR-ing E8Q_STATUS_*
 *     bits into `*status_dev` (a device uint32 the caller zeroes beforehand).
 *   - Weights are [batch, rows, cols] row-major; a group is 8 consecutive
 *     columns of one row; cols % 8 == 0; batch*rows*cols < 2^40 and
 *     rows*cols/8 < 2^32.
 *   - Lattice points are reported as 2z (integers): z is in E8 = D8 u (D8+1/2)
 *     iff all 2z_i are even or all odd and sum(2z) = 0 mod 4.
 *   - Calls on different streams may run concurrently; the library keeps no
 *     mutable device state between calls.  Its read-only tables (core ranks,
 *     points, roots) are generated when the library is built and are part of
 *     its device code object: no call allocates, frees, uploads or
 *     synchronizes.
 *
 * Numerics (bit-exact contract; the CPU oracle computes the same):
 *   v = w (float32, bf16 widened exactly)
 *   rotation (optional): v_j <- sign_j * v_j, then for each block of `b`
 *     columns the un-normalized Sylvester Walsh-Hadamard transform in float32,
 *     butterfly stages of stride 1, 2, 4, ..., b/2 in that order, each mapping
 *     (p, q) -> (p + q, p - q); rotated value u = fl32(v * kappa_b),
 *     kappa_b = fl32(1/sqrt(b)) (kappa = 1 without rotation)
 *   c_r = fl32(kappa_b * fl32(1 / s_r)), x = fl32(v * c_r)
 *   nearest E8 point of each group: n = rint(x) (ties to even), a = |x - n|,
 *     sgn_i = +1 if x_i >= n_i else -1; D8 point: n, and if sum(n) is odd
 *     coordinate k (largest a, lowest index) moved by sgn_k; D8+1/2 point:
 *     n + sgn/2, and if sum(2y) != 0 mod 4 coordinate m (smallest a, lowest
 *     index) moved by -sgn_m; the D8 point is taken iff
 *     sum(a) - 2 + [D8 fixed](1 - 2a_k) - [D8+1/2 fixed] 2a_m <= 0, evaluated
 *     exactly as that float64 expression with sum(a) added pairwise
 *     ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7))
 *   q = fl32(s_r * z); bf16 outputs round to nearest even
 *   invalid data: row with !(s_r > 0), s_r = inf or c_r = inf -> every group
 *     z = 0, E8Q_STATUS_BAD_SCALE; group with a non-finite x -> z = 0,
 *     E8Q_STATUS_NONFINITE; group with some |x_i| >= 8192 -> z = 0,
 *     E8Q_STATUS_X_RANGE.  q of a bad row is +0.
 */
#ifndef E8Q_H
#define E8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes (an int32_t, so that any value a caller passes back, e.g. to
 * e8q_status_string, is well-defined). */
typedef int32_t e8q_status_t;
enum {
    E8Q_OK = 0,
    E8Q_ERR_INVALID = 1,
    E8Q_ERR_UNSUPPORTED = 2,
    E8Q_ERR_LAUNCH = 3,
    E8Q_ERR_DEVICE = 4,
    E8Q_ERR_SCRATCH = 5      /* e8q_encode_core_escape_noalloc: input too large for its fixed scratch */
};

/* Bits OR-ed into *status_dev by the kernels. */
enum {
    E8Q_STATUS_NONFINITE = 1u,       /* a group had a NaN/Inf normalized coordinate      */
    E8Q_STATUS_BAD_SCALE = 2u,       /* a row scale was not a positive finite number     */
    E8Q_STATUS_INT8_RANGE = 4u,      /* a 2z value was saturated in an int8 output       */
    E8Q_STATUS_ESC_OVERFLOW = 8u,    /* more escapes than esc_capacity; records cut      */
    E8Q_STATUS_X_RANGE = 16u,        /* a group had |x_i| >= 8192                        */
    E8Q_STATUS_LOOKBACK_TIMEOUT = 32u, /* escape offsets not resolved in time (outputs invalid) */
    E8Q_STATUS_BAD_INDEX = 64u,      /* decode: a core index >= |C(B)| (decoded as 0)    */
    E8Q_STATUS_ESC_MISSING = 128u    /* decode: an escaped slot had no record (decoded as 0) */
};

/* Element type codes (an int32_t: any other value is rejected with E8Q_ERR_INVALID). */
typedef int32_t e8q_dtype_t;
enum { E8Q_F32 = 0, E8Q_BF16 = 1 };

/* One escape record, 20 bytes.  E8-QAT stores groups outside the core exactly
 * as 20-byte coordinate records (Table 10; Figure 6(c): payload 2 + 20 rho
 * bits per weight).  Field layout (a reading; the pages give only the size):
 * the group index within its matrix (row * cols/8 + col/8), then 2z as int16. */
typedef struct {
    uint32_t group;
    int16_t two_z[8];
} e8q_escape_t;

/* A root-packed escape record, 8 bytes: the escaped point is the core point
 * core_idx plus the root number `root` (E8-QAT Table 3: every escaped group of
 * the artifact is a core point plus one root of E8).  Roots are numbered 0..239
 * in lexicographic order of 2r (signed, coordinate 0 first); the root used is
 * the first that brings the point into the core (a reading).  root == 0xFF
 * (core_idx == 0xFFFF): no root does; the full record is in the wide list. */
typedef struct {
    uint32_t group;
    uint16_t core_idx;
    uint8_t root;
    uint8_t pad;         /* 0 */
} e8q_escape_packed_t;

/* ---------------------------------------------------------------------------
 * e8q_project -- forward projection without rotation: q = s * nearest_E8(w/s).
 * E8-QAT abstract and Figure 1(c)/2(b) captions: every forward pass maps each
 * group of eight normalized weights to its nearest E8 point by arithmetic.
 *
 *   w            [batch, rows, cols] weights, dtype w_dtype (F32 or BF16)
 *   row_scale    [batch*rows] float32 reconstruction scale s_r
 *   q_out        [batch, rows, cols] dequantized s*z in q_dtype, or NULL
 *   two_z_out    [batch, rows, cols] int8 2z (saturated, E8Q_STATUS_INT8_RANGE), or NULL
 *   core_bound   with esc_count_out: a group counts as escaped if ||2z||^2 > core_bound (>= 0)
 *   esc_count_out [batch] int64, overwritten with the per-batch-item escape count, or NULL
 *   status_dev   device uint32, bits OR-ed in (required)
 * At least one of q_out, two_z_out, esc_count_out must be non-NULL.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_project(const void* w, e8q_dtype_t w_dtype,
                         int64_t batch, int64_t rows, int64_t cols,
                         const float* row_scale,
                         void* q_out, e8q_dtype_t q_dtype,
                         int8_t* two_z_out,
                         int32_t core_bound, int64_t* esc_count_out,
                         uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_project_hadamard -- e8q_project after a randomized Walsh-Hadamard
 * rotation (E8-QAT Figure 2 caption: Hadamard transforms precede the
 * projection but are not drawn).  Arguments as e8q_project, plus:
 *   signs        [cols] int8, each +1 or -1 (another value is undefined behaviour)
 *   had_block    b: a power of two in [8, 4096] dividing cols
 *   rotated_out  [batch, rows, cols] float32 u = fl32(v * kappa_b), or NULL
 * q = s * z is in the rotated basis.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_project_hadamard(const void* w, e8q_dtype_t w_dtype,
                                  int64_t batch, int64_t rows, int64_t cols,
                                  const float* row_scale,
                                  const int8_t* signs, int32_t had_block,
                                  void* q_out, e8q_dtype_t q_dtype,
                                  int8_t* two_z_out, float* rotated_out,
                                  int32_t core_bound, int64_t* esc_count_out,
                                  uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_project_hadamard_restore -- e8q_project_hadamard with the projection
 * rotated back to the original weight basis, the form a QAT forward feeds to
 * its matmul (E8-QAT Figure 2 caption: the Hadamard transforms surround the
 * projection but are not drawn; undoing the rotation is a reading).
 *   w_hat = R^T (s z) = sigma * fl32(T * c2), T = H_b (2z) (float32
 *   butterflies in the forward stage order, exact for every |2z| <= 2^24 / b),
 *   c2 = fl32(fl32(s * kappa_b) * 0.5); every zero is sigma * (+0).
 * Arguments as e8q_project_hadamard, except:
 *   w_hat_out    [batch, rows, cols] restored weights in w_hat_dtype (F32, or
 *                BF16 rounded to nearest even) (required)
 *   two_z_out, core_bound, esc_count_out   as e8q_project (optional)
 * A row with an invalid scale (E8Q_STATUS_BAD_SCALE) restores to sigma * (+0).
 * Its identity STE is exact: the composite w -> w_hat has Jacobian I through
 * the rounding, so e8q_ste_backward applies unchanged.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_project_hadamard_restore(const void* w, e8q_dtype_t w_dtype,
                                          int64_t batch, int64_t rows, int64_t cols,
                                          const float* row_scale,
                                          const int8_t* signs, int32_t had_block,
                                          void* w_hat_out, e8q_dtype_t w_hat_dtype,
                                          int8_t* two_z_out,
                                          int32_t core_bound, int64_t* esc_count_out,
                                          uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_encode_core_escape -- export encoding (E8-QAT Figure 2(c): core indices
 * plus sparse escape records keep the final lattice points exactly).
 *
 * Core C(B) = { z in E8 : ||2z||^2 <= B } (a reading of the pages' finite
 * core; B = core_bound in [0, 40], |C(40)| = 56,881).  The core index of z is
 * its rank among C(B) sorted lexicographically by 2z (signed, coordinate 0
 * most significant); escaped groups get 0xFFFF.
 *
 *   w, w_dtype, batch, rows, cols, row_scale   as e8q_project
 *   signs        [cols] int8 +-1, or NULL for no rotation (had_block ignored)
 *   had_block    as e8q_project_hadamard when signs != NULL
 *   core_idx_out [batch*rows*cols/8] uint16 (required)
 *   esc_out      [esc_capacity] records, ascending (batch, group); the records
 *                of batch item i start at sum(esc_count_out[0..i-1]).  Records
 *                past esc_capacity are dropped and E8Q_STATUS_ESC_OVERFLOW is
 *                set; esc_out may be NULL only when esc_capacity == 0.
 *   esc_count_out [batch] int64, exact per-batch escape counts (required)
 *   two_z_out    [batch, rows, cols] int8 2z (saturated), or NULL
 *   workspace    device scratch of at least e8q_encode_workspace_size() bytes,
 *                256-byte aligned; contents need no initialization and are
 *                clobbered.  One workspace must not be shared by calls that
 *                may run at the same time.
 * Escape order is deterministic (it does not depend on scheduling).
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_encode_core_escape(const void* w, e8q_dtype_t w_dtype,
                                    int64_t batch, int64_t rows, int64_t cols,
                                    const float* row_scale,
                                    const int8_t* signs, int32_t had_block,
                                    int32_t core_bound,
                                    uint16_t* core_idx_out,
                                    e8q_escape_t* esc_out, int64_t esc_capacity,
                                    int64_t* esc_count_out,
                                    int8_t* two_z_out,
                                    void* workspace, size_t workspace_bytes,
                                    uint32_t* status_dev, void* stream);

/* Workspace bytes e8q_encode_core_escape needs for this shape (0 on bad sizes). */
size_t e8q_encode_workspace_size(int64_t batch, int64_t rows, int64_t cols);

/* ---------------------------------------------------------------------------
 * e8q_encode_core_escape_noalloc -- e8q_encode_core_escape for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments and results
 * without `workspace`; its scratch is a fixed array in the library's device
 * code object, E8Q_ENCODE_NOALLOC_SCRATCH_BYTES per GPU, held from load time
 * until the process ends.  The call allocates and frees nothing.
 *   - Shapes with e8q_encode_workspace_size(batch, rows, cols) above
 *     E8Q_ENCODE_NOALLOC_SCRATCH_BYTES return E8Q_ERR_SCRATCH before anything
 *     is enqueued (64 MiB covers about 6 G weights per call, e.g. 64 matrices
 *     of 11008 x 4096).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     a GPU (different streams, or threads) race and give undefined results;
 *     calls ordered on one stream are fine.  Each call clears what must start
 *     at zero with a kernel (no memset), so stale contents never leak.
 * ------------------------------------------------------------------------- */
#define E8Q_ENCODE_NOALLOC_SCRATCH_BYTES (64u << 20)

e8q_status_t e8q_encode_core_escape_noalloc(const void* w, e8q_dtype_t w_dtype,
                                            int64_t batch, int64_t rows, int64_t cols,
                                            const float* row_scale,
                                            const int8_t* signs, int32_t had_block,
                                            int32_t core_bound,
                                            uint16_t* core_idx_out,
                                            e8q_escape_t* esc_out, int64_t esc_capacity,
                                            int64_t* esc_count_out,
                                            int8_t* two_z_out,
                                            uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_sgd_project_hadamard -- a QAT step's latent update fused with the next
 * forward projection (E8-QAT Figure 2(b) caption: the identity STE hands the
 * gradient to the latent weights, which the next forward projects again;
 * Table 4: BF16 latents).  For every element of the bf16 latents
 *   w <- bf16_RNE(fl32(w) - fl32(lr * g))     (NaN -> 0x7FC0),
 * the rule of e8q_ste_backward, stored in place; then the outputs of
 * e8q_project_hadamard (e8q_project when signs is NULL) for the updated
 * latents, bit for bit.  The latents are read once per step instead of twice.
 *   w_latent    [batch, rows, cols] bf16, read and overwritten (required)
 *   grad        [batch, rows, cols] bf16 gradient dL/dq, passed through the
 *               identity STE as dL/dw (required; may not alias w_latent)
 *   lr          learning rate
 *   row_scale, signs, had_block, q_out, q_dtype, two_z_out, core_bound,
 *   esc_count_out, status_dev, stream   as e8q_project_hadamard (signs NULL:
 *               no rotation, had_block ignored); at least one output
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_sgd_project_hadamard(void* w_latent, const void* grad, float lr,
                                      int64_t batch, int64_t rows, int64_t cols,
                                      const float* row_scale,
                                      const int8_t* signs, int32_t had_block,
                                      void* q_out, e8q_dtype_t q_dtype,
                                      int8_t* two_z_out, int32_t core_bound,
                                      int64_t* esc_count_out,
                                      uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_sgd_project_hadamard_restore -- the same fused step with the projection
 * written back in the original basis: the latent update of
 * e8q_sgd_project_hadamard, then the outputs of e8q_project_hadamard_restore
 * for the updated latents, bit for bit (E8-QAT Figure 2 caption: the
 * transforms surround the projection).
 *   w_latent, grad, lr   as e8q_sgd_project_hadamard
 *   other arguments as e8q_project_hadamard_restore (signs and w_hat_out
 *   required)
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_sgd_project_hadamard_restore(void* w_latent, const void* grad, float lr,
                                              int64_t batch, int64_t rows, int64_t cols,
                                              const float* row_scale,
                                              const int8_t* signs, int32_t had_block,
                                              void* w_hat_out, e8q_dtype_t w_hat_dtype,
                                              int8_t* two_z_out, int32_t core_bound,
                                              int64_t* esc_count_out,
                                              uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_sgd_rotated_project_hadamard -- the fused step for a forward whose
 * output q lives in the rotated basis: the gradient dL/dq is taken back
 * through the rotation exactly as e8q_ste_backward_hadamard does
 * (dL/dw = sigma * fl32(kappa_b H_b g), float32), the latents step with it
 * (w <- bf16_RNE(fl32(w) - fl32(lr * dL/dw)), NaN -> 0x7FC0) in place, and
 * the outputs of e8q_project_hadamard for the updated latents follow, bit for
 * bit the two calls in sequence (E8-QAT Figure 2 caption: the transforms
 * surround the projection; Figure 2(b): the STE).
 *   w_latent, lr   as e8q_sgd_project_hadamard
 *   grad_q         [batch, rows, cols] bf16 gradient with respect to q (required)
 *   other arguments as e8q_project_hadamard (signs required)
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_sgd_rotated_project_hadamard(void* w_latent, const void* grad_q, float lr,
                                              int64_t batch, int64_t rows, int64_t cols,
                                              const float* row_scale,
                                              const int8_t* signs, int32_t had_block,
                                              void* q_out, e8q_dtype_t q_dtype,
                                              int8_t* two_z_out, int32_t core_bound,
                                              int64_t* esc_count_out,
                                              uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_ste_backward -- identity straight-through estimator (E8-QAT Figure 2(b)
 * caption), optionally fused with a plain SGD step on the latent weights
 * (Table 4: latents are BF16).
 *   grad_q    [n] gradient with respect to q, dtype `dtype` (required)
 *   grad_w    [n] receives grad_q bit for bit, or NULL
 *   w_latent  [n] updated in place: w <- fl32(w - fl32(lr * g)), rounded to
 *             nearest even for BF16 (NaN -> 0x7FC0), or NULL
 * At least one of grad_w, w_latent must be non-NULL; grad_w may alias neither.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_ste_backward(const void* grad_q, void* grad_w, void* w_latent,
                              float lr, e8q_dtype_t dtype, int64_t n, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_ste_backward_hadamard -- the identity STE (E8-QAT Figure 2(b) caption)
 * for a projection whose output q stays in the rotated basis: the gradient of
 * the latent weights is R^T dL/dq = sigma * fl32(kappa_b * H_b g) per block
 * (every zero as sigma * (+0)), optionally fused with the SGD step
 * w <- fl32(w - fl32(lr * g_w)) on the float32 g_w.
 *   grad_q    [rows, cols] gradient with respect to q, dtype `dtype` (required)
 *   signs, had_block   the forward's (had_block a power of two in [8, 4096]
 *             dividing cols; cols <= 30720, or 22528 when had_block > 128)
 *   grad_w    [rows, cols] receives g_w in `dtype` (BF16: nearest even, NaN ->
 *             0x7FC0), or NULL; it may be grad_q itself (in place)
 *   w_latent  [rows, cols] updated in place (BF16 rounded as grad_w), or NULL;
 *             it may alias neither grad_q nor grad_w
 * At least one of grad_w, w_latent must be non-NULL.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_ste_backward_hadamard(const void* grad_q, e8q_dtype_t dtype,
                                       int64_t rows, int64_t cols,
                                       const int8_t* signs, int32_t had_block,
                                       void* grad_w, void* w_latent, float lr,
                                       void* stream);

/* ---------------------------------------------------------------------------
 * e8q_decode_core_escape -- the exported form back to lattice points and
 * weights (E8-QAT Figure 2(c) caption: core indices and escape records keep
 * the final lattice points exactly; Table 3: every core codeword decodes the
 * same on each decoding path).
 *
 *   core_idx     [batch*rows*cols/8] uint16 as written by e8q_encode_core_escape
 *   esc, esc_capacity   the records array and how many records it holds
 *                (4-byte aligned; NULL only with esc_capacity == 0)
 *   esc_count    [batch] int64 per-batch escape counts; the records of batch
 *                item i start at the sum of the earlier counts (clipped to
 *                esc_capacity: a list the encoder cut short decodes with
 *                E8Q_STATUS_ESC_MISSING for the groups whose record is gone)
 *   core_bound   the encoder's B
 *   row_scale    [batch*rows] float32 s_r; required with q_out or w_hat_out
 *   signs, had_block   the encoder's rotation; required with w_hat_out
 *   two_z_out    [batch, rows, cols] int8 2z (saturated, E8Q_STATUS_INT8_RANGE), or NULL
 *   q_out        [batch, rows, cols] q = fl32(s z) in the rotated basis (the
 *                projection's dequantization, bit for bit), q_dtype F32 or BF16, or NULL
 *   w_hat_out    [batch, rows, cols] w_hat = R^T (s z) in the original basis
 *                (as e8q_project_hadamard_restore), w_hat_dtype F32 or BF16, or NULL
 *   workspace    device scratch of e8q_decode_workspace_size(batch) bytes,
 *                8-byte aligned; clobbered; not shared by concurrent calls
 * At least one output must be non-NULL.  A slot that holds 0xFFFF takes the
 * record of its group (binary search: the records of a batch item must be in
 * ascending group order, as the encoder writes them); records of slots that
 * are not escaped are ignored.  An index >= |C(B)| other than 0xFFFF decodes
 * to 0 (E8Q_STATUS_BAD_INDEX); an escaped slot with no record decodes to 0
 * (E8Q_STATUS_ESC_MISSING).  A row whose scale is not a positive finite
 * number gives q = +0 and w_hat = sigma * (+0) (E8Q_STATUS_BAD_SCALE).
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_decode_core_escape(const uint16_t* core_idx,
                                    const e8q_escape_t* esc, int64_t esc_capacity,
                                    const int64_t* esc_count,
                                    int64_t batch, int64_t rows, int64_t cols,
                                    int32_t core_bound,
                                    const float* row_scale,
                                    const int8_t* signs, int32_t had_block,
                                    int8_t* two_z_out,
                                    void* q_out, e8q_dtype_t q_dtype,
                                    void* w_hat_out, e8q_dtype_t w_hat_dtype,
                                    void* workspace, size_t workspace_bytes,
                                    uint32_t* status_dev, void* stream);

/* Workspace bytes e8q_decode_core_escape needs (0 on a bad batch count). */
size_t e8q_decode_workspace_size(int64_t batch);

/* ---------------------------------------------------------------------------
 * e8q_gemv_core_escape -- y = W_hat x from the exported form, the product a
 * 2-bit decode step serves (E8-QAT abstract: decode throughput of the 2-bit
 * representation against BF16; Figure 2(c): the exported form).  W_hat is the
 * restored weight matrix of each batch item (as e8q_decode_core_escape's
 * w_hat, before any rounding); it is never formed: with x~ = kappa_b H_b
 * (sigma * x) computed once per activation vector in float32,
 * y_r = (s_r / 2) * sum_g 2z_g . x~_g.
 *   core_idx, esc, esc_capacity, esc_count, core_bound, row_scale, signs,
 *   had_block   as e8q_decode_core_escape (signs NULL: no rotation, W_hat = s z)
 *   x            [batch, m, cols] activations, x_dtype F32 or BF16; m in {1, 2, 4}
 *   y_out        [batch, m, rows] float32
 *   workspace    e8q_gemv_workspace_size(batch, m, rows, cols) bytes, 256-byte aligned
 * Rows whose column count is a multiple of 256, with 16-byte aligned core_idx,
 * run on the matrix cores.  With cores below 4096 points (B < 24) every
 * activation vector is put in fixed point, x~_k ~ N_k 2^(e-30) with
 * N_k = rint(x~_k 2^(30-e)) and 2^(e-1) <= max_k |x~_k| < 2^e, and the row
 * sums sum_g 2z_g . N_g are exact int32 sums on the int8 matrix cores
 * (N as four signed base-256 digits), y = fl32(fl64((s/2) 2^(e-30) sum));
 * a vector holding a NaN or infinity gives NaN rows (E8Q_STATUS_NONFINITE).
 * With larger cores x~ is split into three bfloat16 parts (exact products,
 * float32 sums whose order inside one MFMA is the hardware's).  Either way the
 * escaped slots are added after the row sums, y += (s / 2) * sum of the row's
 * records' 2z . x~ (float32, in record order, in blocks of 32).  Other shapes
 * use float32 FMA chains with the escaped slots in place.  Rounding, on every
 * path: |y - W_hat x| <= 2 (L + G + 66) 2^-24 S_r + s_r sum_g sum_i |z_gi|
 * (2^(e-31) + 2^-120) per output, L = log2(b), G = ceil(cols / 512),
 * S_r = s_r sum_g sum_i |z_gi| xbar_gi, xbar = kappa_b times the block sums
 * of |x| (|x| itself without rotation).
 * Limits: m * cols * 4 <= 96 KiB, batch <= 65535.  Malformed exports and bad
 * scales are flagged as in e8q_decode_core_escape (a bad row gives y = 0).
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_gemv_core_escape(const uint16_t* core_idx,
                                  const e8q_escape_t* esc, int64_t esc_capacity,
                                  const int64_t* esc_count,
                                  int64_t batch, int64_t rows, int64_t cols,
                                  int32_t core_bound,
                                  const float* row_scale,
                                  const int8_t* signs, int32_t had_block,
                                  const void* x, e8q_dtype_t x_dtype, int64_t m,
                                  float* y_out,
                                  void* workspace, size_t workspace_bytes,
                                  uint32_t* status_dev, void* stream);

/* Workspace bytes e8q_gemv_core_escape needs (0 on bad sizes). */
size_t e8q_gemv_workspace_size(int64_t batch, int64_t m, int64_t rows, int64_t cols);

/* ---------------------------------------------------------------------------
 * e8q_pack_escapes -- escape records to root-packed records (E8-QAT Table 3).
 *   esc, n       the 20-byte records (4-byte aligned)
 *   core_bound   the encoder's B
 *   packed_out   [n] packed records, same order (8-byte aligned)
 *   wide_out, wide_capacity   the full records of points no root brings into
 *                the core, in record order; past the capacity they are
 *                dropped and E8Q_STATUS_ESC_OVERFLOW is set
 *   wide_count_out  device int64: how many records needed the wide list
 *   workspace    e8q_pack_workspace_size(n) bytes, 8-byte aligned
 * Payload with packed records: 2 + 8 rho bits per weight (wide records add
 * 20 bytes each).
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_pack_escapes(const e8q_escape_t* esc, int64_t n, int32_t core_bound,
                              e8q_escape_packed_t* packed_out,
                              e8q_escape_t* wide_out, int64_t wide_capacity,
                              int64_t* wide_count_out,
                              void* workspace, size_t workspace_bytes,
                              uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------
 * e8q_unpack_escapes -- the inverse: packed records (and the wide list of
 * wide_count records) back to 20-byte records esc_out[n] in order.  A packed
 * record with root >= 240 (other than 0xFF) or core_idx >= |C(B)| decodes to
 * 2z = 0 (E8Q_STATUS_BAD_INDEX); one that refers past the wide list decodes to
 * 2z = 0 (E8Q_STATUS_ESC_MISSING).  Workspace as e8q_pack_escapes.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_unpack_escapes(const e8q_escape_packed_t* packed, int64_t n,
                                const e8q_escape_t* wide, int64_t wide_count,
                                int32_t core_bound, e8q_escape_t* esc_out,
                                void* workspace, size_t workspace_bytes,
                                uint32_t* status_dev, void* stream);

/* Workspace bytes e8q_pack_escapes / e8q_unpack_escapes need for n records. */
size_t e8q_pack_workspace_size(int64_t n);

/* ---------------------------------------------------------------------------
 * e8q_ptq_init -- PTQ initialization onto the fixed core (E8-QAT Figure 2(a)
 * caption: PTQ initializes the latent weights from a fixed E8 core; Table 9:
 * QAT then starts with no escapes).  Per row: a scale search over
 * s_k = fl32(alphas[k] * base_scale[r]) by the row's squared error, then the
 * finite-core projection at the chosen scale (the nearest E8 point when it is
 * in C(B), else the nearest point of C(B) by exhaustive search; the search
 * compares float64 keys evaluated in a fixed order, ties to the lower core
 * index).  The scale is chosen on the exact rational row errors
 * E_k = sum (kappa v - s_k z)^2 (v the un-normalized rotated row, kappa the
 * float32 1/sqrt(had_block), z the projection at s_k): the smallest wins,
 * ties go to the smaller k, an invalid scale has E = +inf, a row with a
 * non-finite transform has NaN errors, which count as +inf.
 *   w, w_dtype, batch, rows, cols   as e8q_project
 *   base_scale   [batch*rows] float32 s0 (e.g. the row RMS)
 *   alphas       device float32 [n_alpha] candidate multipliers
 *   signs, had_block   rotation (signs NULL: none)
 *   core_bound   B in [0, 40]
 *   scale_out    [batch*rows] float32 chosen scales (required)
 *   choice_out   [batch*rows] int32 chosen k, or NULL
 *   err_out      [batch*rows, n_alpha] float64 row errors, or NULL: each within
 *                relative (cols+2)u/(1-(cols+2)u), u = 2^-53, of the exact
 *                E_k (+inf for an invalid scale, NaN for a non-finite row)
 *   core_idx_out [batch*rows*cols/8] uint16 (required): the exported form with
 *                no escapes; decode it with e8q_decode_core_escape and zero counts
 *   two_z_out    [batch, rows, cols] int8 2z (required)
 *   workspace    e8q_ptq_workspace_size(batch, rows, cols) bytes, 256-aligned
 * Limits: cols <= 52216 (the row's group errors and work list sit in LDS);
 * with a rotation also cols <= 30720 (had_block <= 128) or 22528 (larger
 * blocks); rotation blocks as e8q_project_hadamard.
 * Status bits as the projection at the chosen scale.
 * ------------------------------------------------------------------------- */
e8q_status_t e8q_ptq_init(const void* w, e8q_dtype_t w_dtype,
                          int64_t batch, int64_t rows, int64_t cols,
                          const float* base_scale, const float* alphas, int32_t n_alpha,
                          const int8_t* signs, int32_t had_block, int32_t core_bound,
                          float* scale_out, int32_t* choice_out, double* err_out,
                          uint16_t* core_idx_out, int8_t* two_z_out,
                          void* workspace, size_t workspace_bytes,
                          uint32_t* status_dev, void* stream);

/* Workspace bytes e8q_ptq_init needs (0 on bad sizes). */
size_t e8q_ptq_workspace_size(int64_t batch, int64_t rows, int64_t cols);

/* |C(core_bound)|, the number of core points; -1 if core_bound is outside [0, 40].
 * Host-only. */
int64_t e8q_core_size(int32_t core_bound);

/* Short text for a return code.  Host-only. */
const char* e8q_status_string(e8q_status_t s);

/* Library version string.  Host-only. */
const char* e8q_version(void);

#ifdef __cplusplus
}
#endif

#endif /* E8Q_H */
