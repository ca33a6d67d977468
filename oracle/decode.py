"""Decoding the exported form: core indices and escape records back to lattice
points, dequantized weights in the rotated basis, and restored weights in the
original basis.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E8-QAT keeps the final lattice points exactly in the exported form (core
indices plus sparse escape records) and checks that its decoding paths agree on
every core codeword [E8-QAT, Figure 2(c) caption; Table 3].  The decoder here
is the plain composition of the oracle's pieces: ``pipeline.decode_core_escape``
(2z), ``pipeline.dequantize`` (q = s z) and ``restore.restore_original``
(w_hat = R^T (s z)).
"""

import numpy as np

from .pipeline import (STATUS_INT8_RANGE, _saturate_int8, decode_core_escape, dequantize,
                       f32_to_bf16)
from .restore import restore_original


def decode_outputs(core_idx, records, counts, core_bound, shape, s=None, signs=None,
                   had_block=0, want_two_z=True):
    """Everything the decode kernel can write, for ``shape = (batch, rows, cols)``.

    Returns a dict with ``two_z`` (int64 [G, 8]), ``two_z_i8`` (saturated,
    [batch, rows, cols]), ``q_f32``/``q_bf16`` (when ``s`` is given),
    ``w_hat_f32``/``w_hat_bf16`` (when ``s`` and ``signs`` are given) and
    ``status``.  Rows whose scale is not a positive finite number give +0 in q
    and sigma * (+0) in w_hat.
    """
    batch, rows, cols = shape
    two_z, status = decode_core_escape(core_idx, records, counts, core_bound, with_status=True)
    i8, sat = _saturate_int8(two_z)
    if want_two_z and sat:
        status |= STATUS_INT8_RANGE
    out = {"two_z": two_z, "two_z_i8": i8.reshape(shape)}
    if s is not None:
        q, st = dequantize(two_z, s, shape)
        status |= st
        out["q_f32"] = q
        out["q_bf16"] = f32_to_bf16(q)
        if signs is not None:
            s_rows = np.asarray(s, dtype=np.float32).reshape(batch * rows)
            bad = ~(s_rows > 0) | np.isinf(s_rows)
            wh = restore_original(two_z.reshape(batch * rows, cols), s_rows, signs, had_block, bad)
            out["w_hat_f32"] = wh.reshape(shape)
            out["w_hat_bf16"] = f32_to_bf16(out["w_hat_f32"])
    out["status"] = status
    return out
