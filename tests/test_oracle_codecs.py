"""Pins of the oracle's number formats against closed forms and brute force.

E2M1 (4-bit element) and E4M3 (block scale), as named by "Pretraining Large
Language Models with NVFP4", Technische Zusammenfassung 2.A (16-element blocks,
E4M3 block scales, FP32 tensor scale).  The value sets are those of the OCP
Microscaling formats specification (E2M1) and OCP FP8 (E4M3).
"""
import numpy as np
import pytest

import oracle

# OCP MX E2M1 value set, by code (sign bit 3).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _all_bits_f32(lo, hi, step=1):
    return np.arange(lo, hi, step, dtype=np.uint64).astype(np.uint32).view(np.float32)


def _brute_e2m1(y):
    """argmin over the 8 magnitudes, ties to even code; sign from the sign bit."""
    # any magnitude above 6 is nearest to 6; clipping keeps fp64 distances distinct
    a = np.minimum(np.abs(y.astype(np.float64)), 8.0)
    mags = np.array(E2M1_TABLE)
    d = np.abs(a[:, None] - mags[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer an even code
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    sign = np.signbit(y).astype(np.uint8) << 3
    return (sign | pick.astype(np.uint8)).astype(np.uint8)


def test_e2m1_decode_table():
    for c in range(16):
        mag = E2M1_TABLE[c & 7]
        want = -mag if c & 8 else mag
        got = oracle.e2m1_decode(c)
        assert got == want and np.signbit(got) == bool(c & 8)


def test_e2m1_roundtrip_all_codes():
    # I-1: every code decodes to a value that re-encodes (f = 1) to itself, incl. -0.
    vals = np.array([oracle.e2m1_decode(c) for c in range(16)], np.float32)
    assert list(oracle.e2m1_encode_rne(vals)) == list(range(16))


def test_e2m1_rne_near_every_decision_point():
    # I-2: dense neighbourhoods (+-2^16 ulps) of every midpoint and grid value,
    # both signs, against the brute-force argmin.
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + E2M1_TABLE + [7.0, 8.0]
    ys = []
    for p in pts:
        b = np.float32(p).view(np.uint32).astype(np.int64)
        ys.append(np.arange(max(b - 65536, 0), b + 65536, dtype=np.int64).astype(np.uint32))
    y = np.concatenate(ys).view(np.float32)
    y = np.concatenate([y, -y])
    np.testing.assert_array_equal(oracle.e2m1_encode_rne(y), _brute_e2m1(y))


def test_e2m1_rne_sweep_and_random():
    # Every fp32 in [0, 16) at a stride of 97 ulps, all bf16 patterns, and random values.
    y1 = _all_bits_f32(0, int(np.float32(16.0).view(np.uint32)), 97)
    y2 = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    y2 = y2[np.isfinite(y2)]
    rng = np.random.default_rng(1)
    y3 = (rng.standard_normal(1 << 20) * 4).astype(np.float32)
    y = np.concatenate([y1, -y1, y2, y3])
    np.testing.assert_array_equal(oracle.e2m1_encode_rne(y), _brute_e2m1(y))


def test_e2m1_saturation_and_specials():
    y = np.array([6.0, 6.5, 7.0, 1e30, np.finfo(np.float32).max, -7.0, 0.0, -0.0,
                  1e-45, -1e-45], np.float32)
    got = oracle.e2m1_encode_rne(y)
    assert list(got) == [7, 7, 7, 7, 7, 15, 0, 8, 0, 8]


def _e4m3_positive_values():
    vals = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_e4m3_decode():
    want = _e4m3_positive_values()
    got = np.array([oracle.e4m3_decode(b) for b in range(0x7F)])
    np.testing.assert_array_equal(got, want)
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x38) == 1.0
    assert np.isnan(oracle.e4m3_decode(0x7F))
    assert oracle.e4m3_decode(0xB8) == -1.0


def _brute_e4m3(t):
    vals = _e4m3_positive_values()
    d = np.abs(np.minimum(t.astype(np.float64), 1e6)[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & (np.arange(len(vals))[None, :] % 2 == 0)
    return np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)


def test_e4m3_encode_against_brute_force():
    # I-3: neighbourhoods of every value and every midpoint, a sweep, and saturation.
    vals = _e4m3_positive_values()
    mids = (vals[1:] + vals[:-1]) / 2
    pts = np.concatenate([vals, mids, [448.0, 464.0, 480.0, 1e4]])
    ts = []
    for p in pts:
        b = int(np.float32(p).view(np.uint32))
        ts.append(np.arange(max(b - 4096, 0), b + 4096, dtype=np.int64).astype(np.uint32))
    t = np.concatenate(ts).view(np.float32)
    sweep = _all_bits_f32(0, int(np.float32(1024.0).view(np.uint32)), 1009)
    t = np.concatenate([t, sweep])
    got = oracle.e4m3_encode(t)
    np.testing.assert_array_equal(got, _brute_e4m3(t))
    assert oracle.e4m3_encode(np.array([np.inf, 3e38], np.float32)).tolist() == [0x7E, 0x7E]


def test_e2m1_sr_choices_and_threshold():
    # The SR result is always one of the two neighbours; for a grid value it is that value;
    # the number of draws u in [0, 2^16) that round up is exactly trunc(r * 2^16).
    u = np.arange(65536, dtype=np.uint16)
    rng = np.random.default_rng(2)
    grid = np.array(E2M1_TABLE)
    for a in list(rng.uniform(0, 6, 40)) + [0.0, 0.5, 1.0, 1.75, 3.0, 4.0, 5.999]:
        a = np.float32(a)
        lo_i = int(np.searchsorted(grid, float(a), side="right") - 1)
        lo, hi = grid[lo_i], grid[min(lo_i + 1, 7)]
        codes = oracle.e2m1_encode_sr(np.full(65536, a, np.float32), u)
        assert set(np.unique(codes)).issubset({lo_i, min(lo_i + 1, 7)})
        if a == lo:
            assert (codes == lo_i).all()
            continue
        r = (float(a) - lo) / (hi - lo)
        assert int((codes == lo_i + 1).sum()) == int(np.floor(r * 65536))
        # the up-set is a prefix of the draws: u < P
        ups = codes == lo_i + 1
        assert ups[: int(ups.sum())].all()
    # saturation and sign
    assert oracle.e2m1_encode_sr(np.array([7.0, -7.0, -0.0], np.float32),
                                 np.zeros(3, np.uint16)).tolist() == [7, 15, 8]
