"""Pins for the oracle's root packing of escape records: the root system of E8
(count, norms, membership, symmetry), the packing rule checked point by point
by a plain loop, the exact round trip, and a property of E8 itself: every
point just outside the core C(16) is a core point plus a root."""

import itertools

import numpy as np

import oracle


def test_roots_are_the_240_minimal_vectors():
    r = oracle.e8_roots()
    assert r.shape == (240, 8)
    assert ((r * r).sum(1) == 8).all()
    assert oracle.is_e8_two_z(r).all()
    assert [tuple(v) for v in r] == sorted(tuple(v) for v in r)
    assert len({tuple(v) for v in r}) == 240
    assert {tuple(-v) for v in r} == {tuple(v) for v in r}
    assert ((np.abs(r) == 2).sum(1) == 2).sum() == 112 and (np.abs(r) == 1).all(1).sum() == 128
    # no E8 point other than 0 is shorter: the roots are the minimal vectors
    pts = oracle.core_points(8)
    assert set(map(tuple, pts[(pts * pts).sum(1) > 0])) == set(map(tuple, r))


def _shell(n2):
    """All E8 points with ||2z||^2 == n2 (brute force over the box)."""
    m = int(np.sqrt(n2))
    out = []
    for parity in (0, 1):
        vals = [v for v in range(-m, m + 1) if (v & 1) == parity]
        for t in itertools.product(vals, repeat=8):
            if sum(v * v for v in t) == n2 and sum(t) % 4 == 0:
                out.append(t)
    return np.array(out, dtype=np.int64)


def test_points_just_outside_the_core_pack():
    """Every E8 point with ||2z||^2 = 24 is a point of C(16) plus a root."""
    shell = _shell(24)
    assert len(shell) == 240 * 28        # theta series of E8: 6720 vectors of norm 6
    rec = np.zeros(len(shell), dtype=oracle.ESCAPE_RECORD_DTYPE)
    rec["group"] = np.arange(len(shell))
    rec["two_z"] = shell
    packed, wide = oracle.pack_escapes(rec, 16)
    assert len(wide) == 0


def test_packing_rule_and_round_trip():
    rng = np.random.default_rng(3)
    roots = oracle.e8_roots()
    w = (rng.normal(size=(2, 32, 1024)) * 0.02).astype(np.float32)
    s = oracle.rms_scale(w.reshape(64, 1024), 1.0)
    for bound in (8, 16, 40):
        enc = oracle.encode_core_escape(w, s, None, 0, bound, w_is_bf16=False)
        rec = enc["records"]
        packed, wide = oracle.pack_escapes(rec, bound)
        assert np.array_equal(oracle.unpack_escapes(packed, wide, bound), rec)
        for k in range(0, len(rec), max(1, len(rec) // 200)):
            tz = rec["two_z"][k].astype(np.int64)
            first = None
            for i, r in enumerate(roots):
                if ((tz - r) ** 2).sum() <= bound:
                    first = i
                    break
            if first is None:
                assert packed["root"][k] == oracle.ROOT_NONE and packed["core_idx"][k] == 0xFFFF
            else:
                assert packed["root"][k] == first
                assert packed["core_idx"][k] == oracle.core_rank((tz - roots[first])[None], bound)[0]
        assert len(wide) == (packed["root"] == oracle.ROOT_NONE).sum()
