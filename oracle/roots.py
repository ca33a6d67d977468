"""Root-packed escape records.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E8-QAT checks that every escaped group of its exported artifact differs from a
core point by one root of E8, so that an escape can be stored as a core index
plus a root [E8-QAT, Table 3: single-root membership].  The pages do not say
which core point is used; the reading here: the roots R = {r in E8 :
||r||^2 = 2} (240 of them) are ordered lexicographically by 2r (signed,
coordinate 0 most significant), and an escaped point z is packed with the
first root r in that order for which z - r lies in the core C(B); its record
keeps the group, the core index of z - r and the root's position.  A point with
no such root keeps its full 20-byte record in a separate list, in record order.
"""

import itertools

import numpy as np

from .core import core_rank, core_unrank
from .pipeline import ESCAPE_RECORD_DTYPE

ROOT_NONE = 0xFF

# 8-byte packed record: group, core index of z - r, root position, padding.
PACKED_RECORD_DTYPE = np.dtype([("group", "<u4"), ("core_idx", "<u2"), ("root", "u1"), ("pad", "u1")])


def e8_roots():
    """The 240 roots of E8 as 2r (int64 [240, 8]) in lexicographic order:
    the 112 vectors with two entries +-2 (2r of (+-1, +-1, 0, ...)) and the
    128 vectors of +-1 with an even number of minus signs [SPLAG ch. 4 sec. 8.1]."""
    pts = []
    for i, j in itertools.combinations(range(8), 2):
        for a in (-2, 2):
            for b in (-2, 2):
                v = [0] * 8
                v[i], v[j] = a, b
                pts.append(v)
    for signs in itertools.product((-1, 1), repeat=8):
        if sum(1 for s in signs if s < 0) % 2 == 0:
            pts.append(list(signs))
    pts = sorted(pts)
    return np.array(pts, dtype=np.int64)


def pack_escapes(records, core_bound):
    """Returns ``(packed, wide)``: one ``PACKED_RECORD_DTYPE`` entry per record
    (``root == ROOT_NONE`` and ``core_idx == 0xFFFF`` when no root works) and
    the 20-byte records of those that could not be packed, in order."""
    roots = e8_roots()
    n = len(records)
    packed = np.zeros(n, dtype=PACKED_RECORD_DTYPE)
    packed["group"] = records["group"]
    packed["root"] = ROOT_NONE
    packed["core_idx"] = 0xFFFF
    if n == 0:
        return packed, np.zeros(0, dtype=ESCAPE_RECORD_DTYPE)
    has = np.zeros(n, dtype=bool)
    for lo in range(0, n, 16384):                                  # bounded memory
        tz = records["two_z"][lo:lo + 16384].astype(np.int64)       # [k, 8]
        diff = tz[:, None, :] - roots[None, :, :]                  # [k, 240, 8]
        ok = (diff * diff).sum(-1) <= core_bound
        h = ok.any(1)
        first = np.argmax(ok, axis=1)
        if h.any():
            rows = np.nonzero(h)[0]
            c = diff[rows, first[rows]]
            packed["root"][lo + rows] = first[rows].astype(np.uint8)
            packed["core_idx"][lo + rows] = core_rank(c, core_bound).astype(np.uint16)
        has[lo:lo + len(tz)] = h
    wide = records[~has].copy()
    return packed, wide


def unpack_escapes(packed, wide, core_bound):
    """Inverse of ``pack_escapes``: the 20-byte records in their order."""
    roots = e8_roots()
    n = len(packed)
    out = np.zeros(n, dtype=ESCAPE_RECORD_DTYPE)
    out["group"] = packed["group"]
    p = packed["root"] != ROOT_NONE
    if p.any():
        c = core_unrank(packed["core_idx"][p].astype(np.int64), core_bound)
        out["two_z"][p] = (c + roots[packed["root"][p].astype(np.int64)]).astype(np.int16)
    k = np.nonzero(~p)[0]
    if len(k):
        out["two_z"][k] = wide["two_z"][: len(k)]
    return out
