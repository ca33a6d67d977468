"""Helpers for the GPU parity tests: run the HIP library through its Python
binding and bring results back as numpy arrays in the oracle's formats."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test needs a ROCm device")
    e8q.lib()                     # raises if the HIP library is missing
    return torch.device("cuda:0")


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def wbits(w):
    """Weights as the oracle takes them: bf16 bits (uint16) or float32."""
    if w.dtype == torch.bfloat16:
        return u16(w)
    return w.cpu().numpy()


def run_project(w, s, signs=None, hb=0, q_dtype=torch.bfloat16, two_z=True, rotated=False,
                core_bound=-1):
    d = w.device
    st = torch.zeros(1, dtype=torch.int32, device=d)
    q = torch.empty(w.shape, dtype=q_dtype, device=d) if q_dtype is not None else None
    tz = torch.empty(w.shape, dtype=torch.int8, device=d) if two_z else None
    u = torch.empty(w.shape, dtype=torch.float32, device=d) if rotated else None
    batch = 1 if w.dim() == 2 else w.shape[0]
    esc = torch.empty(batch, dtype=torch.int64, device=d) if core_bound >= 0 else None
    if signs is None:
        e8q.e8q_project(w, s, st, q_out=q, two_z_out=tz, core_bound=core_bound, esc_count_out=esc)
    else:
        e8q.e8q_project_hadamard(w, s, signs, hb, st, q_out=q, two_z_out=tz, rotated_out=u,
                                 core_bound=core_bound, esc_count_out=esc)
    torch.cuda.synchronize()
    out = {"status": int(st.item()) & 0xFFFFFFFF}
    if q is not None:
        out["q"] = u16(q) if q_dtype == torch.bfloat16 else q.cpu().numpy()
    if tz is not None:
        out["two_z_i8"] = tz.cpu().numpy()
    if u is not None:
        out["u"] = u.cpu().numpy()
    if esc is not None:
        out["esc_count"] = esc.cpu().numpy()
    return out


def run_encode(w, s, core_bound, signs=None, hb=0, cap=None, two_z=False, keep_device=False):
    d = w.device
    batch, rows, cols = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    groups = batch * rows * cols // 8
    if cap is None:
        cap = groups
    st = torch.zeros(1, dtype=torch.int32, device=d)
    core = torch.empty(groups, dtype=torch.int16, device=d)
    esc = torch.empty(max(cap, 1) * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=d)
    if cap == 0:
        esc = None
    cnt = torch.empty(batch, dtype=torch.int64, device=d)
    ws = torch.empty(e8q.e8q_encode_workspace_size(batch, rows, cols), dtype=torch.uint8, device=d)
    tz = torch.empty(w.shape, dtype=torch.int8, device=d) if two_z else None
    e8q.e8q_encode_core_escape(w, s, core_bound, core, esc, cnt, ws, st, signs=signs, had_block=hb,
                               two_z_out=tz)
    torch.cuda.synchronize()
    counts = cnt.cpu().numpy()
    n = int(min(counts.sum(), cap))
    rec = (esc[: n * 20].cpu().numpy().view(oracle.ESCAPE_RECORD_DTYPE) if n
           else np.zeros(0, oracle.ESCAPE_RECORD_DTYPE))
    out = {"status": int(st.item()) & 0xFFFFFFFF, "core_idx": u16(core), "counts": counts,
           "records": rec}
    if tz is not None:
        out["two_z_i8"] = tz.cpu().numpy()
    if keep_device:
        out["dev"] = (core, esc, cnt)
    return out


def first_mismatch(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    bad = np.nonzero((a != b).reshape(-1))[0]
    if len(bad) == 0:
        return None
    i = bad[0]
    return f"{len(bad)} mismatches, first at flat {i}: {a.reshape(-1)[i]} vs {b.reshape(-1)[i]}"


def run_restore(w, s, signs, hb, out_dtype=torch.bfloat16, two_z=True, core_bound=-1):
    d = w.device
    st = torch.zeros(1, dtype=torch.int32, device=d)
    wh = torch.empty(w.shape, dtype=out_dtype, device=d)
    tz = torch.empty(w.shape, dtype=torch.int8, device=d) if two_z else None
    batch = 1 if w.dim() == 2 else w.shape[0]
    esc = torch.empty(batch, dtype=torch.int64, device=d) if core_bound >= 0 else None
    e8q.e8q_project_hadamard_restore(w, s, signs, hb, wh, st, two_z_out=tz, core_bound=core_bound,
                                     esc_count_out=esc)
    torch.cuda.synchronize()
    out = {"status": int(st.item()) & 0xFFFFFFFF,
           "w_hat": u16(wh) if out_dtype == torch.bfloat16 else wh.cpu().numpy()}
    if tz is not None:
        out["two_z_i8"] = tz.cpu().numpy()
    if esc is not None:
        out["esc_count"] = esc.cpu().numpy()
    return out


def same_bits_or_nan(a, b):
    """float32 arrays equal bit for bit, except that NaN matches any NaN."""
    a = np.asarray(a, np.float32).reshape(-1)
    b = np.asarray(b, np.float32).reshape(-1)
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return f"NaN positions differ ({na.sum()} vs {nb.sum()})"
    return first_mismatch(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def upload_export(enc, d):
    """The oracle's exported form (core indices, records, counts) as device tensors."""
    core = torch.from_numpy(enc["core_idx"].view(np.int16).copy()).to(d)
    rec = enc["records"]
    esc = torch.from_numpy(rec.view(np.uint8).reshape(-1).copy()).to(d) if len(rec) else None
    cnt = torch.from_numpy(np.asarray(enc["counts"], np.int64).copy()).to(d)
    return core, esc, cnt


def run_decode(core, esc, cnt, shape, bound, s=None, signs=None, hb=0, two_z=True, q_dtype=None,
               w_hat_dtype=None, esc_records=None):
    d = core.device
    batch = shape[0]
    st = torch.zeros(1, dtype=torch.int32, device=d)
    ws = torch.empty(e8q.e8q_decode_workspace_size(batch), dtype=torch.uint8, device=d)
    tz = torch.empty(shape, dtype=torch.int8, device=d) if two_z else None
    q = torch.empty(shape, dtype=q_dtype, device=d) if q_dtype is not None else None
    wh = torch.empty(shape, dtype=w_hat_dtype, device=d) if w_hat_dtype is not None else None
    e8q.e8q_decode_core_escape(core, esc, cnt, shape, bound, ws, st, row_scale=s, signs=signs,
                               had_block=hb, two_z_out=tz, q_out=q, w_hat_out=wh, esc_records=esc_records)
    torch.cuda.synchronize()
    out = {"status": int(st.item()) & 0xFFFFFFFF}
    if tz is not None:
        out["two_z_i8"] = tz.cpu().numpy()
    if q is not None:
        out["q"] = u16(q) if q_dtype == torch.bfloat16 else q.cpu().numpy()
    if wh is not None:
        out["w_hat"] = u16(wh) if w_hat_dtype == torch.bfloat16 else wh.cpu().numpy()
    return out


def run_gemv(core, esc, cnt, shape, bound, s, x, signs=None, hb=0, esc_records=None):
    d = core.device
    batch, rows, cols = shape
    m = x.shape[1]
    st = torch.zeros(1, dtype=torch.int32, device=d)
    ws = torch.empty(e8q.e8q_gemv_workspace_size(batch, m, rows, cols), dtype=torch.uint8, device=d)
    y = torch.empty((batch, m, rows), dtype=torch.float32, device=d)
    e8q.e8q_gemv_core_escape(core, esc, cnt, shape, bound, s, x, y, ws, st, signs=signs, had_block=hb,
                             esc_records=esc_records)
    torch.cuda.synchronize()
    return {"status": int(st.item()) & 0xFFFFFFFF, "y": y.cpu().numpy().astype(np.float64)}


def gemv_tolerance(two_z, s, x_vals, signs, hb, cols):
    """The documented bound 2 (L + G + 66) 2^-24 S_r + s_r sum|z| (2^(e-30) +
    2^-120) of the GEMV (every evaluation order), e = 1 + the binary exponent
    of the largest xbar of the activation vector (xbar_i >= |x~_i|, so 2^e is
    at least twice the vector's largest |x~|: the int8 kernel's fixed-point
    step is at most 2^(e-31))."""
    L = int(np.log2(hb)) if hb else 0
    G = -(-cols // 512)
    S = oracle.rotated_magnitude(two_z, s, x_vals, signs, hb)
    tz = np.asarray(two_z, dtype=np.float64)
    z1 = np.abs(tz).sum(-1) * 0.5 * np.asarray(s, dtype=np.float64).reshape(tz.shape[0], tz.shape[1])
    xbar = oracle.rotated_bound(x_vals, signs, hb)
    mx = xbar.max(axis=-1)                                   # [batch, m]
    e = np.frexp(np.where(mx > 0, mx, 1.0))[1] + 1
    step = np.where(mx > 0, np.ldexp(1.0, e - 30), 0.0)
    return 2.0 * (L + G + 66) * 2.0 ** -24 * S + (step[:, :, None] + 2.0 ** -120) * z1[:, None, :]


def run_ptq(w, s0, alphas, bound, signs=None, hb=0):
    d = w.device
    batch, rows, cols = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    groups = batch * rows * cols // 8
    st = torch.zeros(1, dtype=torch.int32, device=d)
    al = torch.as_tensor(np.asarray(alphas, np.float32)).to(d)
    scale = torch.empty(batch * rows, dtype=torch.float32, device=d)
    choice = torch.empty(batch * rows, dtype=torch.int32, device=d)
    err = torch.empty((batch * rows, len(alphas)), dtype=torch.float64, device=d)
    core = torch.empty(groups, dtype=torch.int16, device=d)
    tz = torch.empty(w.shape, dtype=torch.int8, device=d)
    ws = torch.empty(e8q.e8q_ptq_workspace_size(batch, rows, cols), dtype=torch.uint8, device=d)
    e8q.e8q_ptq_init(w, s0, al, bound, scale, core, tz, ws, st, signs=signs, had_block=hb, choice_out=choice,
                     err_out=err)
    torch.cuda.synchronize()
    return {"status": int(st.item()) & 0xFFFFFFFF, "scale": scale.cpu().numpy(), "k": choice.cpu().numpy(),
            "err": err.cpu().numpy(), "core_idx": u16(core), "two_z_i8": tz.cpu().numpy(), "dev": (core, scale)}
