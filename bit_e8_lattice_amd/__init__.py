"""bit_e8_lattice_amd -- MI355X (gfx950) E8 lattice projection for E8-QAT.

A thin ctypes binding over ``libe8q.so`` (C ABI in ``include/e8q.h``).  The
Python functions carry the same names as the C entry points and only marshal
arguments: torch tensors supply device memory and the current HIP stream; every
step of the computation runs in the library's HIP kernels.  Nothing here falls
back to the CPU: if the library is missing, calls raise.
"""

import ctypes
import os

import torch

__all__ = [
    "E8QError", "lib", "library_path",
    "e8q_project", "e8q_project_hadamard", "e8q_project_hadamard_restore", "e8q_sgd_project_hadamard",
    "e8q_sgd_project_hadamard_restore", "e8q_sgd_rotated_project_hadamard",
    "e8q_encode_core_escape", "e8q_encode_workspace_size", "e8q_encode_core_escape_noalloc",
    "ENCODE_NOALLOC_SCRATCH_BYTES", "e8q_ste_backward",
    "e8q_ste_backward_hadamard", "e8q_decode_core_escape", "e8q_decode_workspace_size",
    "e8q_gemv_core_escape", "e8q_gemv_workspace_size", "e8q_pack_escapes", "e8q_unpack_escapes",
    "e8q_pack_workspace_size", "PACKED_RECORD_BYTES", "e8q_ptq_init", "e8q_ptq_workspace_size",
    "e8q_core_size",
    "e8q_status_string", "e8q_version",
    "ESCAPE_RECORD_BYTES", "STATUS_BITS", "F32", "BF16",
]

F32, BF16 = 0, 1
ESCAPE_RECORD_BYTES = 20
ENCODE_NOALLOC_SCRATCH_BYTES = 64 << 20      # E8Q_ENCODE_NOALLOC_SCRATCH_BYTES
PACKED_RECORD_BYTES = 8
STATUS_BITS = {
    "NONFINITE": 1, "BAD_SCALE": 2, "INT8_RANGE": 4, "ESC_OVERFLOW": 8,
    "X_RANGE": 16, "LOOKBACK_TIMEOUT": 32, "BAD_INDEX": 64, "ESC_MISSING": 128,
}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libe8q.so")
_lib = None


class E8QError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().e8q_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{fn} failed: {msg} (code {code})")
        self.code = code


def lib():
    """Load ``libe8q.so`` (built in-tree by ``bit_e8_lattice_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is missing: run `python -m bit_e8_lattice_amd.build`")
    L = ctypes.CDLL(library_path)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    e = ctypes.c_int
    L.e8q_project.argtypes = [vp, e, i64, i64, i64, vp, vp, e, vp, i32, vp, vp, vp]
    L.e8q_project.restype = e
    L.e8q_project_hadamard.argtypes = [vp, e, i64, i64, i64, vp, vp, i32, vp, e, vp, vp, i32, vp, vp, vp]
    L.e8q_project_hadamard.restype = e
    L.e8q_project_hadamard_restore.argtypes = [vp, e, i64, i64, i64, vp, vp, i32, vp, e, vp, i32, vp, vp, vp]
    L.e8q_project_hadamard_restore.restype = e
    L.e8q_ste_backward_hadamard.argtypes = [vp, e, i64, i64, vp, i32, vp, vp, f32, vp]
    L.e8q_ste_backward_hadamard.restype = e
    L.e8q_decode_core_escape.argtypes = [vp, vp, i64, vp, i64, i64, i64, i32, vp, vp, i32, vp, vp, e, vp, e,
                                         vp, sz, vp, vp]
    L.e8q_decode_core_escape.restype = e
    L.e8q_decode_workspace_size.argtypes = [i64]
    L.e8q_decode_workspace_size.restype = sz
    L.e8q_gemv_core_escape.argtypes = [vp, vp, i64, vp, i64, i64, i64, i32, vp, vp, i32, vp, e, i64, vp,
                                       vp, sz, vp, vp]
    L.e8q_gemv_core_escape.restype = e
    L.e8q_gemv_workspace_size.argtypes = [i64, i64, i64, i64]
    L.e8q_gemv_workspace_size.restype = sz
    L.e8q_pack_escapes.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp, sz, vp, vp]
    L.e8q_pack_escapes.restype = e
    L.e8q_unpack_escapes.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, vp, vp]
    L.e8q_unpack_escapes.restype = e
    L.e8q_pack_workspace_size.argtypes = [i64]
    L.e8q_pack_workspace_size.restype = sz
    L.e8q_ptq_init.argtypes = [vp, e, i64, i64, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    L.e8q_ptq_init.restype = e
    L.e8q_ptq_workspace_size.argtypes = [i64, i64, i64]
    L.e8q_ptq_workspace_size.restype = sz
    L.e8q_encode_core_escape.argtypes = [vp, e, i64, i64, i64, vp, vp, i32, i32, vp, vp, i64, vp, vp,
                                         vp, sz, vp, vp]
    L.e8q_encode_core_escape.restype = e
    L.e8q_encode_core_escape_noalloc.argtypes = [vp, e, i64, i64, i64, vp, vp, i32, i32, vp, vp, i64, vp, vp,
                                                 vp, vp]
    L.e8q_encode_core_escape_noalloc.restype = e
    L.e8q_encode_workspace_size.argtypes = [i64, i64, i64]
    L.e8q_encode_workspace_size.restype = sz
    L.e8q_sgd_project_hadamard.argtypes = [vp, vp, f32, i64, i64, i64, vp, vp, i32, vp, e, vp, i32, vp, vp, vp]
    L.e8q_sgd_project_hadamard.restype = e
    L.e8q_sgd_project_hadamard_restore.argtypes = [vp, vp, f32, i64, i64, i64, vp, vp, i32, vp, e, vp, i32, vp, vp,
                                                   vp]
    L.e8q_sgd_project_hadamard_restore.restype = e
    L.e8q_sgd_rotated_project_hadamard.argtypes = [vp, vp, f32, i64, i64, i64, vp, vp, i32, vp, e, vp, i32, vp, vp,
                                                   vp]
    L.e8q_sgd_rotated_project_hadamard.restype = e
    L.e8q_ste_backward.argtypes = [vp, vp, vp, f32, e, i64, vp]
    L.e8q_ste_backward.restype = e
    L.e8q_core_size.argtypes = [i32]
    L.e8q_core_size.restype = i64
    L.e8q_status_string.argtypes = [e]
    L.e8q_status_string.restype = ctypes.c_char_p
    L.e8q_version.argtypes = []
    L.e8q_version.restype = ctypes.c_char_p
    _lib = L
    return L


# ------------------------------------------------------------------ marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} dtype {t.dtype} not in {dtypes}")


def _dtype_code(t):
    return BF16 if t.dtype == torch.bfloat16 else F32


def _shape3(w):
    if w.dim() == 2:
        return 1, w.shape[0], w.shape[1]
    if w.dim() == 3:
        return tuple(w.shape)
    raise ValueError("weights must be [rows, cols] or [batch, rows, cols]")


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, code):
    if code != 0:
        raise E8QError(fn, code)


_WDT = (torch.float32, torch.bfloat16)


def e8q_project(w, row_scale, status, q_out=None, two_z_out=None, core_bound=-1,
                esc_count_out=None, stream=None):
    """``e8q_project``: q = s * nearest_E8(w / s) per 8-column group (no rotation)."""
    _dev(w, "w", _WDT); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(q_out, "q_out", _WDT); _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(esc_count_out, "esc_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    b, r, c = _shape3(w)
    code = lib().e8q_project(_ptr(w), _dtype_code(w), b, r, c, _ptr(row_scale), _ptr(q_out),
                             _dtype_code(q_out) if q_out is not None else F32, _ptr(two_z_out),
                             int(core_bound), _ptr(esc_count_out), _ptr(status), _stream(w, stream))
    _check("e8q_project", code)


def e8q_project_hadamard(w, row_scale, signs, had_block, status, q_out=None, two_z_out=None,
                         rotated_out=None, core_bound=-1, esc_count_out=None, stream=None):
    """``e8q_project_hadamard``: sign flip + blockwise Walsh-Hadamard, then project."""
    _dev(w, "w", _WDT); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(signs, "signs", (torch.int8,)); _dev(q_out, "q_out", _WDT)
    _dev(two_z_out, "two_z_out", (torch.int8,)); _dev(rotated_out, "rotated_out", (torch.float32,))
    _dev(esc_count_out, "esc_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    b, r, c = _shape3(w)
    code = lib().e8q_project_hadamard(_ptr(w), _dtype_code(w), b, r, c, _ptr(row_scale), _ptr(signs),
                                      int(had_block), _ptr(q_out),
                                      _dtype_code(q_out) if q_out is not None else F32,
                                      _ptr(two_z_out), _ptr(rotated_out), int(core_bound),
                                      _ptr(esc_count_out), _ptr(status), _stream(w, stream))
    _check("e8q_project_hadamard", code)


def e8q_sgd_project_hadamard(w_latent, grad, lr, row_scale, status, signs=None, had_block=0, q_out=None,
                             two_z_out=None, core_bound=-1, esc_count_out=None, stream=None):
    """``e8q_sgd_project_hadamard``: the identity STE with SGD on the bf16
    latents (in place), then the projection of the updated latents."""
    _dev(w_latent, "w_latent", (torch.bfloat16,)); _dev(grad, "grad", (torch.bfloat16,))
    _dev(row_scale, "row_scale", (torch.float32,)); _dev(signs, "signs", (torch.int8,))
    _dev(q_out, "q_out", _WDT); _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(esc_count_out, "esc_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    if grad.shape != w_latent.shape:
        raise ValueError("grad must have the shape of w_latent")
    b, r, c = _shape3(w_latent)
    code = lib().e8q_sgd_project_hadamard(_ptr(w_latent), _ptr(grad), float(lr), b, r, c, _ptr(row_scale),
                                          _ptr(signs), int(had_block), _ptr(q_out),
                                          _dtype_code(q_out) if q_out is not None else F32,
                                          _ptr(two_z_out), int(core_bound), _ptr(esc_count_out), _ptr(status),
                                          _stream(w_latent, stream))
    _check("e8q_sgd_project_hadamard", code)


def e8q_sgd_rotated_project_hadamard(w_latent, grad_q, lr, row_scale, signs, had_block, status, q_out=None,
                                     two_z_out=None, core_bound=-1, esc_count_out=None, stream=None):
    """``e8q_sgd_rotated_project_hadamard``: the rotated-basis gradient taken
    back through the rotation, SGD on the bf16 latents (in place), then the
    rotated projection of the updated latents."""
    _dev(w_latent, "w_latent", (torch.bfloat16,)); _dev(grad_q, "grad_q", (torch.bfloat16,))
    _dev(row_scale, "row_scale", (torch.float32,)); _dev(signs, "signs", (torch.int8,))
    _dev(q_out, "q_out", _WDT); _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(esc_count_out, "esc_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    if grad_q.shape != w_latent.shape:
        raise ValueError("grad_q must have the shape of w_latent")
    b, r, c = _shape3(w_latent)
    code = lib().e8q_sgd_rotated_project_hadamard(_ptr(w_latent), _ptr(grad_q), float(lr), b, r, c, _ptr(row_scale),
                                                  _ptr(signs), int(had_block), _ptr(q_out),
                                                  _dtype_code(q_out) if q_out is not None else F32,
                                                  _ptr(two_z_out), int(core_bound), _ptr(esc_count_out), _ptr(status),
                                                  _stream(w_latent, stream))
    _check("e8q_sgd_rotated_project_hadamard", code)


def e8q_sgd_project_hadamard_restore(w_latent, grad, lr, row_scale, signs, had_block, w_hat_out, status,
                                     two_z_out=None, core_bound=-1, esc_count_out=None, stream=None):
    """``e8q_sgd_project_hadamard_restore``: the identity STE with SGD on the
    bf16 latents (in place), then the projection of the updated latents
    restored to the original basis (``w_hat_out`` float32 or bf16)."""
    _dev(w_latent, "w_latent", (torch.bfloat16,)); _dev(grad, "grad", (torch.bfloat16,))
    _dev(row_scale, "row_scale", (torch.float32,)); _dev(signs, "signs", (torch.int8,))
    _dev(w_hat_out, "w_hat_out", _WDT); _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(esc_count_out, "esc_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    if w_hat_out is None:
        raise ValueError("w_hat_out is required")
    if grad.shape != w_latent.shape:
        raise ValueError("grad must have the shape of w_latent")
    b, r, c = _shape3(w_latent)
    code = lib().e8q_sgd_project_hadamard_restore(_ptr(w_latent), _ptr(grad), float(lr), b, r, c, _ptr(row_scale),
                                                  _ptr(signs), int(had_block), _ptr(w_hat_out),
                                                  _dtype_code(w_hat_out), _ptr(two_z_out), int(core_bound),
                                                  _ptr(esc_count_out), _ptr(status), _stream(w_latent, stream))
    _check("e8q_sgd_project_hadamard_restore", code)


def e8q_project_hadamard_restore(w, row_scale, signs, had_block, w_hat_out, status, two_z_out=None,
                                 core_bound=-1, esc_count_out=None, stream=None):
    """``e8q_project_hadamard_restore``: the projection rotated back to the
    original basis (``w_hat_out`` float32 or bf16, shaped like ``w``)."""
    _dev(w, "w", _WDT); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(signs, "signs", (torch.int8,)); _dev(w_hat_out, "w_hat_out", _WDT)
    _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(esc_count_out, "esc_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    if w_hat_out is None:
        raise ValueError("w_hat_out is required")
    b, r, c = _shape3(w)
    code = lib().e8q_project_hadamard_restore(_ptr(w), _dtype_code(w), b, r, c, _ptr(row_scale),
                                              _ptr(signs), int(had_block), _ptr(w_hat_out),
                                              _dtype_code(w_hat_out), _ptr(two_z_out), int(core_bound),
                                              _ptr(esc_count_out), _ptr(status), _stream(w, stream))
    _check("e8q_project_hadamard_restore", code)


def e8q_encode_workspace_size(batch, rows, cols):
    return int(lib().e8q_encode_workspace_size(batch, rows, cols))


def e8q_encode_core_escape(w, row_scale, core_bound, core_idx_out, esc_out, esc_count_out,
                           workspace, status, signs=None, had_block=0, two_z_out=None, stream=None):
    """``e8q_encode_core_escape``: core indices (uint16 stored in an int16 tensor)
    plus escape records (``esc_out``: uint8 tensor of 20-byte records)."""
    _dev(w, "w", _WDT); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(signs, "signs", (torch.int8,)); _dev(core_idx_out, "core_idx_out", (torch.int16,))
    _dev(esc_out, "esc_out", (torch.uint8,)); _dev(esc_count_out, "esc_count_out", (torch.int64,))
    _dev(workspace, "workspace", (torch.uint8,)); _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(status, "status", (torch.int32,))
    b, r, c = _shape3(w)
    cap = 0 if esc_out is None else esc_out.numel() // ESCAPE_RECORD_BYTES
    code = lib().e8q_encode_core_escape(_ptr(w), _dtype_code(w), b, r, c, _ptr(row_scale), _ptr(signs),
                                        int(had_block), int(core_bound), _ptr(core_idx_out),
                                        _ptr(esc_out), cap, _ptr(esc_count_out), _ptr(two_z_out),
                                        _ptr(workspace), workspace.numel(), _ptr(status),
                                        _stream(w, stream))
    _check("e8q_encode_core_escape", code)


def e8q_encode_core_escape_noalloc(w, row_scale, core_bound, core_idx_out, esc_out, esc_count_out,
                                   status, signs=None, had_block=0, two_z_out=None, stream=None):
    """``e8q_encode_core_escape_noalloc``: ``e8q_encode_core_escape`` without a
    workspace (the library's fixed per-GPU scratch; calls that overlap on one
    GPU race)."""
    _dev(w, "w", _WDT); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(signs, "signs", (torch.int8,)); _dev(core_idx_out, "core_idx_out", (torch.int16,))
    _dev(esc_out, "esc_out", (torch.uint8,)); _dev(esc_count_out, "esc_count_out", (torch.int64,))
    _dev(two_z_out, "two_z_out", (torch.int8,)); _dev(status, "status", (torch.int32,))
    b, r, c = _shape3(w)
    cap = 0 if esc_out is None else esc_out.numel() // ESCAPE_RECORD_BYTES
    code = lib().e8q_encode_core_escape_noalloc(_ptr(w), _dtype_code(w), b, r, c, _ptr(row_scale), _ptr(signs),
                                                int(had_block), int(core_bound), _ptr(core_idx_out),
                                                _ptr(esc_out), cap, _ptr(esc_count_out), _ptr(two_z_out),
                                                _ptr(status), _stream(w, stream))
    _check("e8q_encode_core_escape_noalloc", code)


def e8q_ste_backward(grad_q, grad_w=None, w_latent=None, lr=1.0, stream=None):
    """``e8q_ste_backward``: identity STE copy and/or fused SGD on the latents."""
    _dev(grad_q, "grad_q", _WDT); _dev(grad_w, "grad_w", (grad_q.dtype,))
    _dev(w_latent, "w_latent", (grad_q.dtype,))
    code = lib().e8q_ste_backward(_ptr(grad_q), _ptr(grad_w), _ptr(w_latent), float(lr),
                                  _dtype_code(grad_q), grad_q.numel(), _stream(grad_q, stream))
    _check("e8q_ste_backward", code)


def e8q_ste_backward_hadamard(grad_q, signs, had_block, grad_w=None, w_latent=None, lr=1.0, stream=None):
    """``e8q_ste_backward_hadamard``: gradient of the latents for a rotated-basis
    projection (R^T applied to ``grad_q``), and/or the fused SGD step."""
    _dev(grad_q, "grad_q", _WDT); _dev(signs, "signs", (torch.int8,))
    _dev(grad_w, "grad_w", (grad_q.dtype,)); _dev(w_latent, "w_latent", (grad_q.dtype,))
    cols = grad_q.shape[-1]
    rows = grad_q.numel() // cols
    code = lib().e8q_ste_backward_hadamard(_ptr(grad_q), _dtype_code(grad_q), rows, cols, _ptr(signs),
                                           int(had_block), _ptr(grad_w), _ptr(w_latent), float(lr),
                                           _stream(grad_q, stream))
    _check("e8q_ste_backward_hadamard", code)


def e8q_decode_workspace_size(batch):
    return int(lib().e8q_decode_workspace_size(batch))


def e8q_decode_core_escape(core_idx, esc, esc_count, shape, core_bound, workspace, status, row_scale=None,
                           signs=None, had_block=0, two_z_out=None, q_out=None, w_hat_out=None,
                           esc_records=None, stream=None):
    """``e8q_decode_core_escape``: core indices (int16 tensor of uint16 values)
    and escape records (uint8 tensor of 20-byte records) back to 2z, q
    (rotated basis) and/or w_hat (original basis), for ``shape = (batch, rows,
    cols)``.  ``esc_records`` overrides the record count taken from ``esc``."""
    _dev(core_idx, "core_idx", (torch.int16,)); _dev(esc, "esc", (torch.uint8,))
    _dev(esc_count, "esc_count", (torch.int64,)); _dev(workspace, "workspace", (torch.uint8,))
    _dev(status, "status", (torch.int32,)); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(signs, "signs", (torch.int8,)); _dev(two_z_out, "two_z_out", (torch.int8,))
    _dev(q_out, "q_out", _WDT); _dev(w_hat_out, "w_hat_out", _WDT)
    b, r, c = shape
    cap = 0 if esc is None else esc.numel() // ESCAPE_RECORD_BYTES
    if esc_records is not None:
        cap = min(cap, int(esc_records))
    code = lib().e8q_decode_core_escape(
        _ptr(core_idx), _ptr(esc), cap, _ptr(esc_count), b, r, c, int(core_bound), _ptr(row_scale),
        _ptr(signs), int(had_block), _ptr(two_z_out), _ptr(q_out),
        _dtype_code(q_out) if q_out is not None else F32, _ptr(w_hat_out),
        _dtype_code(w_hat_out) if w_hat_out is not None else F32, _ptr(workspace), workspace.numel(),
        _ptr(status), _stream(core_idx, stream))
    _check("e8q_decode_core_escape", code)


def e8q_gemv_workspace_size(batch, m, rows, cols):
    return int(lib().e8q_gemv_workspace_size(batch, m, rows, cols))


def e8q_gemv_core_escape(core_idx, esc, esc_count, shape, core_bound, row_scale, x, y_out, workspace, status,
                         signs=None, had_block=0, esc_records=None, stream=None):
    """``e8q_gemv_core_escape``: ``y_out[b, t, r] = sum_c W_hat[b, r, c] x[b, t, c]``
    from the exported form, for ``shape = (batch, rows, cols)`` and ``x``
    [batch, m, cols]."""
    _dev(core_idx, "core_idx", (torch.int16,)); _dev(esc, "esc", (torch.uint8,))
    _dev(esc_count, "esc_count", (torch.int64,)); _dev(row_scale, "row_scale", (torch.float32,))
    _dev(x, "x", _WDT); _dev(y_out, "y_out", (torch.float32,)); _dev(workspace, "workspace", (torch.uint8,))
    _dev(status, "status", (torch.int32,)); _dev(signs, "signs", (torch.int8,))
    b, r, c = shape
    if x.dim() != 3 or x.shape[0] != b or x.shape[2] != c:
        raise ValueError("x must be [batch, m, cols]")
    cap = 0 if esc is None else esc.numel() // ESCAPE_RECORD_BYTES
    if esc_records is not None:
        cap = min(cap, int(esc_records))
    code = lib().e8q_gemv_core_escape(
        _ptr(core_idx), _ptr(esc), cap, _ptr(esc_count), b, r, c, int(core_bound), _ptr(row_scale), _ptr(signs),
        int(had_block), _ptr(x), _dtype_code(x), x.shape[1], _ptr(y_out), _ptr(workspace), workspace.numel(),
        _ptr(status), _stream(core_idx, stream))
    _check("e8q_gemv_core_escape", code)


def e8q_pack_workspace_size(n):
    return int(lib().e8q_pack_workspace_size(n))


def e8q_pack_escapes(esc, n, core_bound, packed_out, wide_out, wide_count_out, workspace, status, stream=None):
    """``e8q_pack_escapes``: ``n`` 20-byte records in ``esc`` (uint8 tensor) to
    8-byte packed records in ``packed_out`` (uint8) plus the wide list."""
    for t, nm in ((esc, "esc"), (packed_out, "packed_out"), (wide_out, "wide_out"), (workspace, "workspace")):
        _dev(t, nm, (torch.uint8,))
    _dev(wide_count_out, "wide_count_out", (torch.int64,)); _dev(status, "status", (torch.int32,))
    cap = 0 if wide_out is None else wide_out.numel() // ESCAPE_RECORD_BYTES
    code = lib().e8q_pack_escapes(_ptr(esc), int(n), int(core_bound), _ptr(packed_out), _ptr(wide_out), cap,
                                  _ptr(wide_count_out), _ptr(workspace), workspace.numel(), _ptr(status),
                                  _stream(workspace, stream))
    _check("e8q_pack_escapes", code)


def e8q_unpack_escapes(packed, n, wide, wide_count, core_bound, esc_out, workspace, status, stream=None):
    """``e8q_unpack_escapes``: packed records (+ ``wide_count`` wide records) back to
    20-byte records in ``esc_out`` (uint8)."""
    for t, nm in ((packed, "packed"), (wide, "wide"), (esc_out, "esc_out"), (workspace, "workspace")):
        _dev(t, nm, (torch.uint8,))
    _dev(status, "status", (torch.int32,))
    code = lib().e8q_unpack_escapes(_ptr(packed), int(n), _ptr(wide), int(wide_count), int(core_bound),
                                    _ptr(esc_out), _ptr(workspace), workspace.numel(), _ptr(status),
                                    _stream(workspace, stream))
    _check("e8q_unpack_escapes", code)


def e8q_ptq_workspace_size(batch, rows, cols):
    return int(lib().e8q_ptq_workspace_size(batch, rows, cols))


def e8q_ptq_init(w, base_scale, alphas, core_bound, scale_out, core_idx_out, two_z_out, workspace, status,
                 signs=None, had_block=0, choice_out=None, err_out=None, stream=None):
    """``e8q_ptq_init``: per-row scale search over ``alphas * base_scale`` and the
    finite-core projection at the chosen scale."""
    _dev(w, "w", _WDT); _dev(base_scale, "base_scale", (torch.float32,)); _dev(alphas, "alphas", (torch.float32,))
    _dev(scale_out, "scale_out", (torch.float32,)); _dev(core_idx_out, "core_idx_out", (torch.int16,))
    _dev(two_z_out, "two_z_out", (torch.int8,)); _dev(workspace, "workspace", (torch.uint8,))
    _dev(status, "status", (torch.int32,)); _dev(signs, "signs", (torch.int8,))
    _dev(choice_out, "choice_out", (torch.int32,)); _dev(err_out, "err_out", (torch.float64,))
    b, r, c = _shape3(w)
    code = lib().e8q_ptq_init(_ptr(w), _dtype_code(w), b, r, c, _ptr(base_scale), _ptr(alphas), alphas.numel(),
                              _ptr(signs), int(had_block), int(core_bound), _ptr(scale_out), _ptr(choice_out),
                              _ptr(err_out), _ptr(core_idx_out), _ptr(two_z_out), _ptr(workspace),
                              workspace.numel(), _ptr(status), _stream(w, stream))
    _check("e8q_ptq_init", code)


def e8q_core_size(core_bound):
    return int(lib().e8q_core_size(int(core_bound)))


def e8q_status_string(code):
    return lib().e8q_status_string(int(code)).decode()


def e8q_version():
    return lib().e8q_version().decode()
