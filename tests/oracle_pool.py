"""Forked CPU-oracle workers for full-size parity checks.

The pool must be started before anything in the process touches the GPU (a
process that has initialised HIP must not fork): ``conftest.py`` starts it
right after collection when GPU tests are selected.  Workers only run numpy
and the oracle; inputs reach them pickled, row chunk by row chunk, so host
memory stays bounded.  This module imports neither torch nor the HIP library.
"""

import multiprocessing as mp
import os

import numpy as np

_POOL = None
_WORKERS = 0


def start(workers=None):
    """Fork the workers (idempotent).  At most 16: the host share of one GPU."""
    global _POOL, _WORKERS
    if _POOL is None:
        _WORKERS = workers or max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = mp.get_context("fork").Pool(_WORKERS)
    return _POOL


def stop():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL = None


def pool():
    if _POOL is None:
        raise RuntimeError("oracle pool not started (it must be forked before the GPU is used)")
    return _POOL


def _encode_chunk(job):
    import oracle
    w, s, signs, hb, bound = job
    r = oracle.encode_core_escape(w, s, signs, hb, bound)
    return r["core_idx"], r["records"], int(r["counts"][0]), r["status"]


def _project_chunk(job):
    import oracle
    w, s, signs, hb, bound = job
    r = oracle.project(w, s, signs, hb, core_bound=bound)
    return r["q_bf16"], r["two_z_i8"], int(r["esc_count"][0]), r["status"]


def _chunks(rows, chunk_rows):
    return [(lo, min(rows, lo + chunk_rows)) for lo in range(0, rows, chunk_rows)]


def encode_matrix_async(w, s, signs, hb, bound, chunk_rows=256):
    """Start the oracle encode of one matrix (``w`` [rows, cols] bf16 bits,
    ``s`` [rows]) over row chunks; returns a handle for ``encode_result``."""
    rows = w.shape[0]
    parts = _chunks(rows, chunk_rows)
    jobs = [(np.ascontiguousarray(w[lo:hi]), np.ascontiguousarray(s[lo:hi]), signs, hb, bound) for lo, hi in parts]
    return parts, w.shape[1] // 8, pool().map_async(_encode_chunk, jobs, chunksize=1)


def encode_result(handle):
    """Core indices, records (groups relative to the matrix, ascending), count
    and status of one matrix, assembled from its chunks."""
    parts, gpr, res = handle
    out = res.get()
    core = np.concatenate([o[0] for o in out])
    recs = []
    for (lo, _), o in zip(parts, out):
        r = o[1].copy()
        r["group"] += np.uint32(lo * gpr)
        recs.append(r)
    records = np.concatenate(recs) if recs else np.zeros(0, dtype=out[0][1].dtype)
    status = 0
    for o in out:
        status |= o[3]
    return core, records, sum(o[2] for o in out), status


def project_matrix(w, s, signs, hb, bound, chunk_rows=256):
    """Oracle projection of one matrix: (q bf16 bits [rows, cols], 2z int8
    [rows, cols], escape count, status)."""
    parts = _chunks(w.shape[0], chunk_rows)
    jobs = [(np.ascontiguousarray(w[lo:hi]), np.ascontiguousarray(s[lo:hi]), signs, hb, bound) for lo, hi in parts]
    out = pool().map(_project_chunk, jobs, chunksize=1)
    q = np.concatenate([o[0].reshape(-1, w.shape[1]) for o in out])
    tz = np.concatenate([o[1].reshape(-1, w.shape[1]) for o in out])
    status = 0
    for o in out:
        status |= o[3]
    return q, tz, sum(o[2] for o in out), status


def escape_count_async(w, s, signs, hb, bound, chunk_rows=256):
    """Start the oracle's escape count (||2z||^2 > bound) of one matrix."""
    parts = _chunks(w.shape[0], chunk_rows)
    jobs = [(np.ascontiguousarray(w[lo:hi]), np.ascontiguousarray(s[lo:hi]), signs, hb, bound) for lo, hi in parts]
    return pool().map_async(_escape_chunk, jobs, chunksize=1)


def _escape_chunk(job):
    import oracle
    w, s, signs, hb, bound = job
    return int(oracle.project(w, s, signs, hb, core_bound=bound, want_two_z=False)["esc_count"][0])
