"""The E8-QAT weight path, step by step, in plain numpy.

Steps (the readings of open points are stated where they are used):

1. widen: bf16 weights to float32 (exact);
2. optional randomized Hadamard rotation (``hadamard.fwht_blocks``) after a
   per-column sign flip; rotated output ``u = fl32(v * kappa_b)``
   [E8-QAT, Figure 2 caption: Hadamard transforms are part of the method but
   not drawn];
3. normalize: ``x = fl32(v * c_r)`` with ``c_r = fl32(kappa_b * fl32(1 / s_r))``,
   ``s_r`` the per-row reconstruction scale [E8-QAT, Figure 1(c) caption:
   eight normalized coordinates; Figure 2 caption: reconstruction scales].
   Multiplying by a rounded reciprocal (not dividing per element) is a reading;
4. nearest E8 point of each group of 8 consecutive columns
   (``lattice.nearest_e8_two_z``) [E8-QAT, abstract; Figure 2(b) caption];
5. dequantize ``q = fl32(s_r * z)`` (float32, or bf16 by round-to-nearest-even);
6. core test ``||2z||^2 <= B``, dense core index, escape records for the rest,
   compacted in ascending (batch, group) order with exact per-batch counts
   [E8-QAT, abstract; Figure 2(c) caption; Table 10: 20-byte records];
7. identity straight-through backward and a plain SGD step on bf16 latent
   weights [E8-QAT, Figure 2(b) caption; Table 4: latent weights in BF16].

Invalid data (a reading; the pages never meet it): a row whose scale is not a
positive finite number, or whose coefficient ``c_r`` overflows, maps every
group to ``z = 0`` and sets ``STATUS_BAD_SCALE``; a group with a non-finite
normalized coordinate maps to ``z = 0`` (``STATUS_NONFINITE``); a group with a
coordinate of magnitude >= 2^13 maps to ``z = 0`` (``STATUS_X_RANGE``) so that
every stored ``2z`` fits an int16 escape field.  Such groups count as core.
"""

import numpy as np

from .core import ESCAPE_SLOT, core_rank, core_size, core_unrank
from .hadamard import fwht_blocks, kappa
from .lattice import nearest_e8_two_z

STATUS_NONFINITE = 1
STATUS_BAD_SCALE = 2
STATUS_INT8_RANGE = 4
STATUS_ESC_OVERFLOW = 8
STATUS_X_RANGE = 16

STATUS_BAD_INDEX = 64
STATUS_ESC_MISSING = 128

X_LIMIT = np.float32(8192.0)

# 20-byte escape record: group index within its matrix, then 2z as int16.
# The pages fix only the size [E8-QAT, Table 10]; the field layout is a reading.
ESCAPE_RECORD_DTYPE = np.dtype([("group", "<u4"), ("two_z", "<i2", (8,))])


# --------------------------------------------------------------------------- bf16

def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) to float32: the bits are the top half."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(f):
    """float32 to bf16 bits, round to nearest even; every NaN becomes 0x7FC0."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = rounded.astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), out)


# ------------------------------------------------------------------- normalization

def rms_scale(w_f32, alpha=1.0):
    """Per-row scale ``fl32(alpha * sqrt(mean_j w_rj^2))`` in float64.

    The reconstruction scale is left open by the pages [E8-QAT, Figure 2
    caption]; per-row RMS times a multiplier is the reading used for the
    synthetic workloads.  Used to pin the workload generator.
    """
    w = np.asarray(w_f32, dtype=np.float64)
    r = np.sqrt(np.mean(w * w, axis=-1))
    return (alpha * r).astype(np.float32)


def row_coefficients(s, had_block):
    """``c_r = fl32(kappa_b * fl32(1 / s_r))`` and the bad-row mask."""
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = np.float32(1.0) / s
        c = kappa(had_block) * inv
    bad = ~(s > 0) | np.isinf(s) | np.isinf(c)
    return c.astype(np.float32), bad


def _shape3(w):
    shp = np.asarray(w).shape
    return (1,) + tuple(shp) if len(shp) == 2 else tuple(shp)


def _widen(w, w_is_bf16):
    return bf16_to_f32(w) if w_is_bf16 else np.asarray(w, dtype=np.float32)


def normalized_groups(w, s, signs=None, had_block=0, w_is_bf16=True):
    """Steps 1-3.  ``w``: [batch, rows, cols] (bf16 bits or float32).

    Returns ``(x [G, 8] float32, u or None [batch, rows, cols], bad_row [G] bool,
    row [G] int64)`` where G = batch*rows*cols/8 in memory order.
    """
    v = _widen(w, w_is_bf16)
    if v.ndim == 2:
        v = v[None]
    batch, rows, cols = v.shape
    if cols % 8:
        raise ValueError("cols must be a multiple of 8")
    u = None
    b = 0
    if signs is not None:
        b = int(had_block)
        v = v * np.asarray(signs, dtype=np.int8).astype(np.float32)   # exact
        v = fwht_blocks(v, b)
        u = v * kappa(b)
    c, bad = row_coefficients(np.asarray(s, dtype=np.float32).reshape(batch * rows), b)
    with np.errstate(over="ignore", invalid="ignore"):
        x = v.reshape(batch * rows, cols) * c[:, None]
    gpr = cols // 8
    row = np.repeat(np.arange(batch * rows), gpr)
    return x.reshape(-1, 8), u, bad[row], row


def _lattice_points(x, bad_row):
    """Step 4 with the invalid-data rules.  Returns (2z int64 [G,8], status)."""
    status = 0
    finite = np.isfinite(x).all(axis=1)
    with np.errstate(invalid="ignore"):
        small = (np.abs(np.where(np.isfinite(x), x, 0)) < X_LIMIT).all(axis=1)
    valid = ~bad_row & finite & small
    if bad_row.any():
        status |= STATUS_BAD_SCALE
    if (~bad_row & ~finite).any():
        status |= STATUS_NONFINITE
    if (~bad_row & finite & ~small).any():
        status |= STATUS_X_RANGE
    two_z = np.zeros(x.shape, dtype=np.int64)
    if valid.any():
        two_z[valid] = nearest_e8_two_z(x[valid])
    return two_z, status


def _saturate_int8(two_z):
    out = np.clip(two_z, -128, 127).astype(np.int8)
    return out, bool((out != two_z).any())


# ------------------------------------------------------------------------ project

def project(w, s, signs=None, had_block=0, w_is_bf16=True, core_bound=-1,
            want_two_z=True):
    """Forward projection (steps 1-5) as used in every QAT forward pass.

    Returns a dict with ``two_z`` (int64 [G,8], unsaturated), ``two_z_i8``,
    ``q_f32`` and ``q_bf16`` ([batch, rows, cols]), ``u`` (rotated values or
    None), ``esc_count`` (int64 [batch] groups with ||2z||^2 > core_bound, or
    None when core_bound < 0) and ``status``.
    """
    x, u, bad_row, row = normalized_groups(w, s, signs, had_block, w_is_bf16)
    batch, rows, cols = _shape3(w)
    two_z, status = _lattice_points(x, bad_row)
    s_rows = np.asarray(s, dtype=np.float32).reshape(batch * rows)
    z = (two_z.astype(np.float32) * np.float32(0.5))
    with np.errstate(over="ignore", invalid="ignore"):
        q = s_rows[row][:, None] * z
    q = np.where(bad_row[:, None], np.float32(0.0), q).astype(np.float32)
    q = q.reshape(batch, rows, cols)
    two_z_i8, sat = _saturate_int8(two_z)
    if want_two_z and sat:
        status |= STATUS_INT8_RANGE
    esc = None
    if core_bound >= 0:
        esc_g = (two_z * two_z).sum(axis=1) > core_bound
        esc = esc_g.reshape(batch, -1).sum(axis=1).astype(np.int64)
    return {
        "two_z": two_z,
        "two_z_i8": two_z_i8.reshape(batch, rows, cols),
        "q_f32": q,
        "q_bf16": f32_to_bf16(q),
        "u": u,
        "esc_count": esc,
        "status": status,
    }


# ------------------------------------------------------------------------ encode

def encode_core_escape(w, s, signs=None, had_block=0, core_bound=16,
                       w_is_bf16=True, esc_capacity=None, want_two_z=False):
    """Export encoding (steps 1-4 and 6).

    Returns a dict with ``core_idx`` (uint16 [G], 0xFFFF for escapes),
    ``records`` (``ESCAPE_RECORD_DTYPE`` array, ascending (batch, group), cut at
    ``esc_capacity``), ``counts`` (int64 [batch], exact), ``two_z`` and
    ``status``.
    """
    x, _, bad_row, _ = normalized_groups(w, s, signs, had_block, w_is_bf16)
    batch = _shape3(w)[0]
    two_z, status = _lattice_points(x, bad_row)
    g_total = two_z.shape[0]
    gpb = g_total // batch
    norm = (two_z * two_z).sum(axis=1)
    esc = norm > core_bound
    core_idx = np.full(g_total, ESCAPE_SLOT, dtype=np.uint16)
    if (~esc).any():
        r = core_rank(two_z[~esc], core_bound)
        assert (r >= 0).all()
        core_idx[~esc] = r.astype(np.uint16)
    flat = np.nonzero(esc)[0]
    counts = np.bincount(flat // gpb, minlength=batch).astype(np.int64)
    rec = np.zeros(len(flat), dtype=ESCAPE_RECORD_DTYPE)
    rec["group"] = (flat % gpb).astype(np.uint32)
    rec["two_z"] = two_z[flat].astype(np.int16)
    if esc_capacity is not None and len(rec) > esc_capacity:
        rec = rec[:esc_capacity]
        status |= STATUS_ESC_OVERFLOW
    if want_two_z:
        _, sat = _saturate_int8(two_z)
        if sat:
            status |= STATUS_INT8_RANGE
    return {"core_idx": core_idx, "records": rec, "counts": counts,
            "two_z": two_z, "status": status}


def decode_core_escape(core_idx, records, counts, core_bound, with_status=False):
    """Rebuild every ``2z`` from core indices and escape records
    [E8-QAT, Figure 2(c) caption; Table 3: core decoding agreement].

    Records of batch item ``b`` are ``records[off_b : off_b + counts[b]]`` with
    ``off`` the exclusive prefix sum of ``counts`` (only the records actually
    present count: a list cut short by the encoder's capacity is shorter).  A
    slot holding ``ESCAPE_SLOT`` takes the record of its group; a record whose
    slot is not ``ESCAPE_SLOT`` is ignored.  Malformed input (a reading): an
    index ``>= |C(B)|`` decodes to 0 and sets ``STATUS_BAD_INDEX``; an escape
    slot with no record decodes to 0 and sets ``STATUS_ESC_MISSING``.
    """
    core_idx = np.asarray(core_idx, dtype=np.uint16)
    counts = np.asarray(counts, dtype=np.int64)
    batch = len(counts)
    g_total = core_idx.shape[0]
    gpb = g_total // batch
    out = np.zeros((g_total, 8), dtype=np.int64)
    status = 0
    n_core = core_size(core_bound)
    esc_slot = core_idx == ESCAPE_SLOT
    ok = ~esc_slot & (core_idx.astype(np.int64) < n_core)
    if (~esc_slot & ~ok).any():
        status |= STATUS_BAD_INDEX
    out[ok] = core_unrank(core_idx[ok].astype(np.int64), core_bound)
    off = np.concatenate([[0], np.cumsum(counts)])
    have = np.zeros(g_total, dtype=bool)
    for b in range(batch):
        r = records[min(off[b], len(records)):min(off[b + 1], len(records))]
        gid = b * gpb + r["group"].astype(np.int64)
        inside = (r["group"].astype(np.int64) < gpb)
        gid, r = gid[inside], r[inside]
        take = esc_slot[gid]
        out[gid[take]] = r["two_z"][take].astype(np.int64)
        have[gid[take]] = True
    if (esc_slot & ~have).any():
        status |= STATUS_ESC_MISSING
    return (out, status) if with_status else out


def dequantize(two_z, s, shape):
    """``q = fl32(s_r * z)`` from ``2z`` (the projection's dequantization);
    rows whose scale is not a positive finite number give +0 and
    ``STATUS_BAD_SCALE``.  Returns (q float32 [shape], status)."""
    batch, rows, cols = shape
    s_rows = np.asarray(s, dtype=np.float32).reshape(batch * rows)
    bad = ~(s_rows > 0) | np.isinf(s_rows)
    gpr = cols // 8
    row = np.repeat(np.arange(batch * rows), gpr)
    z = np.asarray(two_z).reshape(-1, 8).astype(np.float32) * np.float32(0.5)
    with np.errstate(over="ignore", invalid="ignore"):
        q = s_rows[row][:, None] * z
    q = np.where(bad[row][:, None], np.float32(0.0), q).astype(np.float32)
    return q.reshape(shape), (STATUS_BAD_SCALE if bad.any() else 0)


# ---------------------------------------------------------------- backward / SGD

def ste_backward(grad_q):
    """Identity straight-through estimator: dL/dw = dL/dq, bit for bit
    [E8-QAT, Figure 2(b) caption]."""
    return np.array(grad_q, copy=True)


def sgd_update(w, g, lr, is_bf16=True):
    """Plain SGD on the latent weights: ``w <- fl32(w - fl32(lr * g))``, rounded
    to bf16 (nearest even) when the latents are bf16 [E8-QAT, Table 4]."""
    wf = _widen(w, is_bf16)
    gf = _widen(g, is_bf16)
    with np.errstate(over="ignore", invalid="ignore"):
        step = np.float32(lr) * gf
        new = (wf - step).astype(np.float32)
    return f32_to_bf16(new) if is_bf16 else new


# ------------------------------------------------------------------- accounting

def escape_fraction(n_escaped_groups, n_groups):
    """rho: escaped groups over all groups (the denominator is groups, which is
    what makes E8-QAT Tables 3, 4 and 9 agree)."""
    return float(n_escaped_groups) / float(n_groups)


def payload_bits(rho, record_bytes=20, index_bits=16, group=8):
    """Bits per weight of index plus extension: a 16-bit index per 8-weight
    group plus one ``record_bytes`` record per escaped group, i.e. 2 + 20 rho
    for 20-byte records [E8-QAT, Figure 6(c) caption; Table 10]."""
    return (index_bits + 8 * record_bytes * rho) / group
