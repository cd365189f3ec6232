"""Pins: the oracle against an exact-rational brute force on tiny tensors.

tests/exact_model.py models every binary32 step with exact rationals and
finds every code by searching the whole code table, so an operand swapped,
a term dropped, a wrong index or a wrong tie rule in the oracle shows up as
a mismatch here. Tensors are a few blocks of each data family, for every
recipe, metric, error precision, bound, scale granularity and block shape.
"""
import itertools
import math
import zlib

import numpy as np
import pytest
import torch

import exact_model
import synthdata
from synthdata import raw_bits

MODES = [("nvfp4", "mse", "exact")] + [("4over6", m, p) for m in ("mae", "mse") for p in ("exact", "fp16")]


def _values(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float32).numpy().astype(np.float64)


def _data(family, dtype, M, K, seed):
    if family == "weight":
        t = synthdata.weight(M, K, seed, dtype)
    else:
        t = synthdata.activation_family(family, M, K, seed, dtype)
    if family == "outlier":  # make sure the tiny tensor holds outliers
        t = t.clone()
        t.view(-1)[::37] = t.view(-1)[::37] * 1000
    return t


def _amax(orc, t, dtype, gran, block, caller_scale):
    bits = raw_bits(t)
    mode = "tensor" if gran == "tensor" else ("band16" if block == "16x16" else "row")
    a = orc.amax(bits, dtype, mode)
    return (a * np.float32(caller_scale)).astype(np.float32)


CASES = []
for dtype, family, block, gran, bound in itertools.product(
        ("bf16", "fp16", "fp32"), ("normal", "outlier", "special", "weight"), ("1x16", "16x16"),
        ("tensor", "row"), (448, 256)):
    CASES.append((dtype, family, block, gran, bound))


@pytest.mark.parametrize("dtype,family,block,gran,bound", CASES)
def test_oracle_matches_exact_model(orc, dtype, family, block, gran, bound):
    M, K = (2, 32) if block == "1x16" else (16, 32)
    seed = zlib.crc32(repr((dtype, family, block, gran, bound)).encode()) % 1000
    t = _data(family, dtype, M, K, seed)
    # caller amax: the true amax, or a third of it (so scales saturate) for bound 256
    amax = _amax(orc, t, dtype, gran, block, 1.0 if bound == 448 else 1.0 / 3.0)
    bits = raw_bits(t)
    xv = _values(t)
    for recipe, metric, prec in MODES:
        got = orc.quantize(bits, dtype, amax, debug=True, recipe=recipe, block=block, scale_gran=gran,
                           err_metric=metric, err_prec=prec, bound=bound)
        codes, scales, kept, errs = exact_model.quantize_tensor(xv, amax, block, gran, bound, recipe, metric,
                                                                prec)
        np.testing.assert_array_equal(got["codes"], codes, err_msg=f"{recipe} {metric} {prec}")
        np.testing.assert_array_equal(got["scales"], scales, err_msg=f"{recipe} {metric} {prec}")
        np.testing.assert_array_equal(got["choice"], kept)
        if recipe == "4over6":
            np.testing.assert_array_equal(got["err"].astype(np.float64), errs)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("family", ["normal", "outlier", "special", "weight"])
@pytest.mark.parametrize("gran", ["tensor", "row"])
def test_sequential_order_matches_exact_model(orc, dtype, family, gran):
    """The sequential error order (1x16) against the exact model's left fold,
    every mode and bound."""
    M, K = 3, 48
    seed = zlib.crc32(repr(("seq", dtype, family, gran)).encode()) % 1000
    t = _data(family, dtype, M, K, seed)
    bits = raw_bits(t)
    xv = _values(t)
    for bound in (448, 256):
        amax = _amax(orc, t, dtype, gran, "1x16", 1.0 if bound == 448 else 1.0 / 3.0)
        for recipe, metric, prec in MODES:
            got = orc.quantize(bits, dtype, amax, debug=True, recipe=recipe, scale_gran=gran, err_metric=metric,
                               err_prec=prec, bound=bound, err_order="seq")
            codes, scales, kept, errs = exact_model.quantize_tensor(xv, amax, "1x16", gran, bound, recipe, metric,
                                                                    prec, order="seq")
            np.testing.assert_array_equal(got["codes"], codes, err_msg=f"{recipe} {metric} {prec}")
            np.testing.assert_array_equal(got["scales"], scales)
            np.testing.assert_array_equal(got["choice"], kept)
            if recipe == "4over6":
                np.testing.assert_array_equal(got["err"].astype(np.float64), errs)


def test_sequential_order_changes_some_choices(orc):
    """On the outlier family the two orders disagree on some candidate errors,
    so the knob is exercised; 16x16 blocks reject the sequential order."""
    t = synthdata.activation_family("outlier", 64, 512, 9, "bf16")
    bits = raw_bits(t)
    a = orc.amax(bits, "bf16", "tensor")
    kw = dict(recipe="4over6", err_metric="mse", err_prec="exact")
    tr = orc.quantize(bits, "bf16", a, debug=True, err_order="tree", **kw)
    sq = orc.quantize(bits, "bf16", a, debug=True, err_order="seq", **kw)
    assert not np.array_equal(tr["err"], sq["err"])
    with pytest.raises(ValueError):
        orc.quantize(raw_bits(synthdata.weight(16, 32, 1, "bf16")), "bf16", a, block="16x16", err_order="seq")


@pytest.mark.parametrize("metric,prec", [("mse", "fp16"), ("mae", "fp16")])
def test_fp16_error_mode_exercised(orc, metric, prec):
    """On weights with a non-dyadic global scale the binary16 rounding of the
    decoded values changes some candidate errors, and the oracle follows the
    exact model there too."""
    t = synthdata.weight(4, 256, 3, "bf16")
    bits = raw_bits(t)
    amax = orc.amax(bits, "bf16", "tensor") * np.float32(1.37)
    xv = _values(t)
    got_x = orc.quantize(bits, "bf16", amax, debug=True, recipe="4over6", err_metric=metric, err_prec="exact")
    got_h = orc.quantize(bits, "bf16", amax, debug=True, recipe="4over6", err_metric=metric, err_prec=prec)
    assert not np.array_equal(got_x["err"], got_h["err"])
    codes, scales, kept, errs = exact_model.quantize_tensor(xv, amax, "1x16", "tensor", 448, "4over6", metric, prec)
    np.testing.assert_array_equal(got_h["codes"], codes)
    np.testing.assert_array_equal(got_h["err"].astype(np.float64), errs)


def test_specials_match_exact_model(orc):
    """NaN, +-inf, +-0, subnormal and saturating inputs."""
    f = np.float32
    rows = [
        [np.nan, 1, -2, 3, 0, -0.0, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14],
        [np.inf, 1, -2, 3, 0, -0.0, 5, 6, 7, 8, 9, 10, 11, 12, 13, -np.inf],
        [1e-40, -1e-41, 1e-39, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 2e-40],
        [-np.nan, -np.nan] + [0.0] * 14,
        [3e38, -3e38, 1, 2] + [0.5] * 12,
    ]
    x = np.array(rows, f)
    xv = x.astype(np.float64)
    for A in (np.float32(14.0), np.float32(0.0), np.float32(np.inf), np.float32(3e38), np.float32(1e-30)):
        amax = np.array([A], f)
        for recipe, metric, prec in MODES:
            got = orc.quantize(x, "fp32", amax, debug=True, recipe=recipe, err_metric=metric, err_prec=prec)
            codes, scales, kept, errs = exact_model.quantize_tensor(xv, amax, "1x16", "tensor", 448, recipe,
                                                                    metric, prec)
            np.testing.assert_array_equal(got["codes"], codes, err_msg=f"A={A} {recipe} {metric} {prec}")
            np.testing.assert_array_equal(got["scales"], scales, err_msg=f"A={A} {recipe}")
            np.testing.assert_array_equal(got["choice"], kept)
            if recipe == "4over6":
                ge = got["err"].astype(np.float64)
                assert np.array_equal(np.isnan(ge), np.isnan(errs))
                np.testing.assert_array_equal(ge[~np.isnan(ge)], errs[~np.isnan(errs)])


def _order_sensitive_blocks(c: int, n_want: int = 4):
    """Block amaxes a and global amaxes A (bound 448) for which the block
    scale t = RN(RN(a / c) * S_enc) of R-4 and the other association
    a * RN(S_enc / c) round to different E4M3 codes: a is placed a few ulps
    from a midpoint between two E4M3 values, scaled by S_enc. Returns a list
    of (a, A)."""
    rng = np.random.default_rng(100 + c)
    vals = torch.arange(0, 0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (vals[1:] + vals[:-1]) / 2
    A = rng.uniform(1.0, 1000.0, 20000).astype(np.float32)
    S = (np.float32(2688.0) / A).astype(np.float32)
    m = mids[rng.integers(8, mids.size, A.size)]
    a0 = (m * c / S.astype(np.float64)).astype(np.float32)
    out = []
    for k in range(-4, 5):
        a = (a0.view(np.int32) + k).view(np.float32)
        t1 = ((a / np.float32(c)).astype(np.float32) * S).astype(np.float32)
        t2 = (a * (S / np.float32(c)).astype(np.float32)).astype(np.float32)
        e1 = torch.from_numpy(np.minimum(t1, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        e2 = torch.from_numpy(np.minimum(t2, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        for i in np.nonzero((e1 != e2) & (a <= A))[0]:
            out.append((float(a[i]), float(A[i])))
    assert len(out) >= n_want, "no order-sensitive blocks found"
    return out[:n_want]


def test_block_scale_rounding_order(orc):
    """R-4 pinned where it matters: on blocks whose map-to-6 scale depends on
    the association of RN(a / 6) * S_enc, the oracle's scale equals the exact
    model's (which takes t = RN(RN(a / 6) * S_enc)). For the map-to-4
    candidate both associations agree: division by 4 is exact."""
    c, recipe = 6, "nvfp4"
    for a, A in _order_sensitive_blocks(c):
        row = np.array([a] + [a * 0.5 ** (i % 7 + 1) for i in range(15)], np.float32).reshape(1, 16)
        amax = np.array([A], np.float32)
        got = orc.quantize(row, "fp32", amax, recipe=recipe)
        codes, scales, _, _ = exact_model.quantize_tensor(row.astype(np.float64), amax, "1x16", "tensor", 448,
                                                          recipe, "mse", "exact")
        np.testing.assert_array_equal(got["scales"], scales, err_msg=f"a={a!r} A={A!r}")
        np.testing.assert_array_equal(got["codes"], codes)


def test_exact_model_rounding_sanity():
    # the model's own binary32 rounding against numpy's float32 cast on random rationals
    rng = np.random.default_rng(1)
    for _ in range(2000):
        a = float(np.float32(rng.standard_normal() * 10.0 ** rng.integers(-40, 38)))
        b = float(np.float32(rng.standard_normal() * 10.0 ** rng.integers(-3, 3)))
        with np.errstate(all="ignore"):
            assert exact_model.mul(a, b) == float(np.float32(a) * np.float32(b)) or \
                math.isinf(exact_model.mul(a, b))
            assert exact_model.add(a, b) == float(np.float32(a) + np.float32(b))
            if b != 0:
                assert exact_model.div(a, b) == float(np.float32(a) / np.float32(b)) or \
                    math.isinf(exact_model.div(a, b))
