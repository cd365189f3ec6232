"""Pins for the oracle's element formats and roundings (CPU only).

The oracle's E2M1/E4M3 code tables, its RNE-with-saturation casts and its
binary16/bfloat16 roundings are checked against things outside the oracle:
the grids the OCP Microscaling Formats spec v1.0 lists, torch's float8_e4m3fn
decode and cast, numpy's float16 cast, torch's bfloat16 cast, and threshold
tables worked out by hand from the round-to-nearest-even rule.
"""
import math

import numpy as np
import pytest
import torch

# E2M1 magnitudes as the OCP MX v1.0 spec tabulates them (codes 0..7).
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

# Hand-worked E2M1 decision points for |v| (ties go to the even code):
# (value, code) pairs at, just below and just above every midpoint.
E2M1_MIDPOINTS = [(0.25, 0, 1), (0.75, 1, 2), (1.25, 2, 3), (1.75, 3, 4), (2.5, 4, 5), (3.5, 5, 6), (5.0, 6, 7)]


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def test_e2m1_grid_matches_ocp(orc):
    for code in range(16):
        mag = OCP_E2M1[code & 7]
        want = -mag if code & 8 else mag
        got = orc.e2m1_value(code)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_grid_matches_torch_decode(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = orc.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, float(ref[c])), c
    # OCP MX v1.0 E4M3 facts: max normal 448, min normal 2^-6, min subnormal 2^-9, NaN at S.1111.111
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))


def test_e2m1_hand_thresholds(orc):
    vals, want = [], []
    for mid, lo, hi in E2M1_MIDPOINTS:
        even = lo if lo % 2 == 0 else hi
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(10))
        vals += [below, np.float32(mid), above]
        want += [lo, even, hi]
    for v, w in list(zip(vals, want)):
        vals.append(-v)
        want.append(w | 8)
    got = orc.e2m1_rne_sat(np.array(vals, np.float32))
    assert got.tolist() == want


def test_e2m1_specials(orc):
    inf = np.float32(np.inf)
    cases = [
        (0.0, 0x0), (-0.0, 0x8), (6.0, 0x7), (7.0, 0x7), (100.0, 0x7), (-1e30, 0xF), (float(inf), 0x7),
        (float(-inf), 0xF), (float(np.float32(1e-45)), 0x0), (-float(np.float32(1e-45)), 0x8),
    ]
    v = np.array([c[0] for c in cases], np.float32)
    assert orc.e2m1_rne_sat(v).tolist() == [c[1] for c in cases]
    # NaN of either sign encodes to +6 (code 0x7)
    nans = _f32([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF])
    assert orc.e2m1_rne_sat(nans).tolist() == [0x7] * 4


def _e2m1_by_midpoints(v):
    """Nearest E2M1 code by searching the sorted midpoints; an exact tie
    goes to the even code of the two neighbours."""
    grid = np.array(OCP_E2M1)
    mids = (grid[:-1] + grid[1:]) / 2
    mag = np.minimum(np.abs(v.astype(np.float64)), 6.0)
    idx = np.searchsorted(mids, mag, side="left")
    tie = (idx < len(mids)) & (mids[np.minimum(idx, len(mids) - 1)] == mag)
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def test_e2m1_all_binary32_in_working_range(orc):
    """Every binary32 value with |v| in [2^-4, 8), both signs, plus every
    bfloat16 and float16 value."""
    chunk = 1 << 22
    lo = np.float32(2.0 ** -4).view(np.uint32)
    hi = np.float32(8.0).view(np.uint32)
    for start in range(int(lo), int(hi), chunk):
        bits = np.arange(start, min(start + chunk, int(hi)), dtype=np.uint32)
        for sgn in (0, 0x80000000):
            v = (bits | np.uint32(sgn)).view(np.float32)
            np.testing.assert_array_equal(orc.e2m1_rne_sat(v), _e2m1_by_midpoints(v))
    h = np.arange(65536, dtype=np.uint32)
    for v in ((h << 16).view(np.float32), h.astype(np.uint16).view(np.float16).astype(np.float32)):
        finite = ~np.isnan(v)
        np.testing.assert_array_equal(orc.e2m1_rne_sat(v[finite]), _e2m1_by_midpoints(v[finite]))


def _e4m3_probe_points():
    """Every E4M3 value and every midpoint between neighbours, each with its
    64 binary32 neighbours on either side, plus 2M random values in [0, 448]."""
    vals = torch.arange(0, 0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    grid = vals.to(torch.float64).numpy()
    pts = np.concatenate([grid, (grid[:-1] + grid[1:]) / 2]).astype(np.float32)
    offs = np.arange(-64, 65, dtype=np.int64)
    bits = pts.view(np.uint32).astype(np.int64)[:, None] + offs[None, :]
    bits = bits[(bits >= 0)].astype(np.uint32)
    dense = bits.view(np.float32)
    rng = np.random.default_rng(7)
    rand = rng.uniform(0, 448, size=2_000_000).astype(np.float32)
    v = np.concatenate([dense, rand])
    return v[(v >= 0) & (v <= 448)]


def test_e4m3_matches_torch_cast(orc):
    v = _e4m3_probe_points()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_rne_sat(v), ref)


def test_e4m3_saturation_and_zero(orc):
    v = np.array([448.0, 448.5, 463.9, 464.0, 500.0, 1e30, np.inf, 0.0, 2.0 ** -10, 2.0 ** -10 + 2.0 ** -30,
                  np.float32(1e-45)], np.float32)
    # 2^-10 is the midpoint between 0 and 2^-9: the tie goes to even code 0x00
    assert orc.e4m3_rne_sat(v).tolist() == [0x7E] * 7 + [0x00, 0x00, 0x01, 0x00]
    assert orc.e4m3_rne_sat(np.array([np.nan], np.float32)).tolist() == [0x7F]


def _f16_probe_points():
    h = np.arange(0x7C00, dtype=np.uint16)  # every finite non-negative binary16
    f = h.view(np.float16).astype(np.float64)
    nxt = np.append(f[1:], 65536.0)
    mids = ((f + nxt) / 2).astype(np.float32)  # exact in binary32
    base = np.concatenate([f.astype(np.float32), mids])
    b = base.view(np.uint32).astype(np.int64)
    pts = np.concatenate([b + d for d in (-2, -1, 0, 1, 2)])
    pts = pts[pts >= 0].astype(np.uint32)
    rng = np.random.default_rng(11)
    rnd = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    allb = np.concatenate([pts, pts | np.uint32(0x80000000), rnd])
    v = allb.view(np.float32)
    return v[~np.isnan(v)]


def test_f16_rounding_matches_numpy(orc):
    v = _f16_probe_points()
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_f16_bits(v), ref)
    assert orc.f32_to_f16_bits(np.array([np.nan, -np.nan], np.float32)).tolist() == [0x7E00, 0x7E00]


def test_bf16_rounding_matches_torch(orc):
    h = np.arange(0x7F80, dtype=np.uint32)
    f = (h << 16).view(np.float32).astype(np.float64)
    nxt = np.append(f[1:], 2.0 ** 128)
    mids = ((f + nxt) / 2)
    mids = mids[mids < 3.4e38].astype(np.float32)
    base = np.concatenate([f.astype(np.float32), mids])
    b = base.view(np.uint32).astype(np.int64)
    pts = np.concatenate([b + d for d in (-2, -1, 0, 1, 2)])
    pts = pts[(pts >= 0) & (pts < 0x7F800000)].astype(np.uint32)
    rng = np.random.default_rng(12)
    rnd = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    allb = np.concatenate([pts, pts | np.uint32(0x80000000), rnd])
    v = allb.view(np.float32)
    v = v[~np.isnan(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_bf16_bits(v), ref)
    assert orc.f32_to_bf16_bits(np.array([np.nan], np.float32)).tolist() == [0x7FC0]


@pytest.mark.parametrize("A,B,want", [
    (2688.0, 448, 1.0), (1536.0, 256, 1.0), (1.0, 448, 2688.0), (1.0, 256, 1536.0), (3.0, 448, 896.0),
    (7.0, 448, 384.0), (0.0, 448, 1.0), (-0.0, 448, 1.0), (float("inf"), 448, 1.0), (float("nan"), 256, 1.0),
    (1e-38, 448, float(np.finfo(np.float32).max)), (float(np.float32(1e-45)), 256, float(np.finfo(np.float32).max)),
])
def test_global_encode_scale_closed_forms(orc, A, B, want):
    assert orc.global_encode_scale(A, B) == np.float32(want)


def test_global_decode_scale_is_reciprocal(orc):
    for A, B in [(3.0, 448), (5.5, 256), (1234.5, 448), (0.0, 448)]:
        s = np.float32(orc.global_encode_scale(A, B))
        assert orc.global_decode_scale(A, B) == np.float32(np.float64(1.0) / np.float64(s))


def _shuffle_down_lane0(u):
    """A model of the mechanism the kernel page describes: sixteen lanes, a
    shuffle-down by 8, 4, 2, 1 where a lane whose source would fall outside
    the 16-lane segment reads its own value (clamped), each lane adding what
    it read to its value in binary32. Returns lane 0."""
    lanes = [np.float32(x) for x in u]
    for off in (8, 4, 2, 1):
        read = [lanes[i + off] if i + off < 16 else lanes[i] for i in range(16)]
        lanes = [np.float32(lanes[i] + read[i]) for i in range(16)]
    return lanes[0]


def test_tree16_exact_value(orc):
    # one 1.0 and fifteen 2^-24: a sequential sum stays 1.0, the tree gives 1 + 7 * 2^-23
    u = np.array([1.0] + [2.0 ** -24] * 15, np.float32)
    assert orc.tree16(u) == np.float32(1.0 + 7 * 2.0 ** -23)
    seq = np.float32(0)
    for x in u:
        seq = np.float32(seq + x)
    assert seq == np.float32(1.0)


def test_seq16_exact_values(orc):
    """The sequential order in closed form: one 1.0 then fifteen 2^-24 stays
    1.0 (each addition is a tie that rounds back to the even 1.0); the same
    terms reversed sum exactly to 15 * 2^-24 first, and 1 + 7.5 ulp rounds to
    the even 1 + 8 ulp = 1 + 2^-20."""
    u = np.array([1.0] + [2.0 ** -24] * 15, np.float32)
    assert orc.seq16(u) == np.float32(1.0)
    assert orc.seq16(u[::-1].copy()) == np.float32(1.0 + 2.0 ** -20)
    # all terms equal to 2^-3: every partial sum is exact
    assert orc.seq16(np.full(16, 0.125, np.float32)) == np.float32(2.0)
    # 2^24 then fifteen ones: sequentially each 2^24 + 1 is a tie that stays
    # at the even 2^24. The tree: stride 8 gives lane 0 2^24 + 1 -> 2^24 and
    # lanes 1..7 the value 2; stride 4: 2^24 + 2, 4, 4, 4; stride 2:
    # 2^24 + 6, 8; stride 1: 2^24 + 14 (all exact past the first tie).
    v = np.array([2.0 ** 24] + [1.0] * 15, np.float32)
    assert orc.seq16(v) == np.float32(2.0 ** 24)
    assert orc.tree16(v) == np.float32(2.0 ** 24 + 14.0)


def test_tree16_matches_shuffle_down_model(orc):
    rng = np.random.default_rng(5)
    for _ in range(3000):
        u = (rng.standard_normal(16) * 2.0 ** rng.integers(-30, 30, 16)).astype(np.float32) ** 2
        assert orc.tree16(u) == _shuffle_down_lane0(u)
