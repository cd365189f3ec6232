"""An exact-rational model of one quantization block, for brute-force pins.

Written independently of the oracle: binary32 arithmetic is modelled by
rounding exact rationals (``fractions.Fraction``) to binary32 with ties to
even, E4M3 block scales are found by searching all 127 finite non-negative
codes (decoded by torch's float8_e4m3fn), E2M1 codes by searching the eight
OCP grid magnitudes, and binary16 rounding uses numpy's float16 cast. The
error sum follows a lane-by-lane model of a clamped shuffle-down over sixteen
lanes, or (the sequential order) a left-to-right sum. It is slow and meant
for a handful of blocks.
"""
from __future__ import annotations

import math
from fractions import Fraction as F

import numpy as np
import torch

OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E4M3_VALUES = torch.arange(0, 0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
    .to(torch.float64).tolist()
FLT_MAX = float(np.finfo(np.float32).max)


def _pow2(e: int) -> F:
    return F(2 ** e) if e >= 0 else F(1, 2 ** (-e))


def rn32(q: F, negative: bool) -> float:
    """Round the exact value q to binary32 (ties to even, gradual underflow,
    overflow to infinity). ``negative`` gives the sign of a zero result."""
    if q == 0:
        return -0.0 if negative else 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _pow2(e) > a:
        e -= 1
    qe = max(e, -126) - 23
    n = a / _pow2(qe)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * _pow2(qe)
    if r >= _pow2(128):
        return sign * math.inf
    if r == 0:
        return sign * 0.0
    return sign * float(r)


def _neg(x: float) -> bool:
    return math.copysign(1.0, x) < 0


def mul(a: float, b: float) -> float:
    if math.isnan(a) or math.isnan(b):
        return math.nan
    if math.isinf(a) or math.isinf(b):
        if a == 0 or b == 0:
            return math.nan
        return math.copysign(math.inf, 1.0 if _neg(a) == _neg(b) else -1.0)
    return rn32(F(a) * F(b), _neg(a) != _neg(b))


def div(a: float, b: float) -> float:
    assert b != 0 and not math.isnan(b) and not math.isinf(b)
    if math.isnan(a):
        return math.nan
    if math.isinf(a):
        return math.copysign(math.inf, 1.0 if _neg(a) == _neg(b) else -1.0)
    return rn32(F(a) / F(b), _neg(a) != _neg(b))


def add(a: float, b: float) -> float:
    if math.isnan(a) or math.isnan(b):
        return math.nan
    if math.isinf(a) or math.isinf(b):
        if math.isinf(a) and math.isinf(b) and _neg(a) != _neg(b):
            return math.nan
        return a if math.isinf(a) else b
    return rn32(F(a) + F(b), _neg(a) and _neg(b))


def sub(a: float, b: float) -> float:
    return add(a, -b)


def lane_tree(terms):
    """Sixteen lanes, shuffle-down by 8, 4, 2, 1 with clamped sources; lane 0."""
    lanes = list(terms)
    for off in (8, 4, 2, 1):
        lanes = [add(lanes[i], lanes[i + off] if i + off < 16 else lanes[i]) for i in range(16)]
    return lanes[0]


def left_fold(terms):
    """Left-to-right sum in element order, each addition rounded."""
    s = terms[0]
    for t in terms[1:]:
        s = add(s, t)
    return s


def nearest_e4m3(t: float) -> int:
    if t >= 448.0:
        return 0x7E
    best, best_d = None, None
    for k, val in enumerate(E4M3_VALUES):
        d = abs(F(t) - F(val))
        if best is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return best


def nearest_e2m1(v: float) -> int:
    if math.isnan(v):
        return 0x7
    sign = 8 if _neg(v) else 0
    m = min(abs(v), 6.0)
    best, best_d = None, None
    for k, g in enumerate(OCP_E2M1):
        d = abs(F(m) - F(g))
        if best is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return sign | best


def e2m1_value(code: int) -> float:
    mag = OCP_E2M1[code & 7]
    return -mag if code & 8 else mag


def global_scales(A: float, bound: int):
    if A > 0 and not math.isinf(A):
        s = div(6.0 * bound, A)
        s = min(s, FLT_MAX)
    else:
        s = 1.0
    return s, div(1.0, s)


def quantize_block(xs, nrows: int, A: float, bound: int, recipe: str, metric: str, prec: str, order: str = "tree"):
    """xs: 16 * nrows binary32 values (row-major). Returns (codes, scale, kept, err6, err4)."""
    S_enc, S_dec = global_scales(A, bound)
    a = 0.0
    for x in xs:
        if not math.isnan(x) and abs(x) > a:
            a = abs(x)
    divisors = {"nvfp4": [6], "4over6": [6, 4], "map4": [4]}[recipe]
    results = {}
    for c in divisors:
        t = mul(div(a, float(c)), S_enc)
        k = nearest_e4m3(t)
        sigma = E4M3_VALUES[k]
        E = 0.0 if sigma == 0 else min(div(S_enc, sigma), FLT_MAX)
        D = mul(sigma, S_dec)
        codes, terms = [], []
        for x in xs:
            q = nearest_e2m1(mul(x, E))
            codes.append(q)
            xhat = mul(e2m1_value(q), D)
            with np.errstate(over="ignore"):
                ref = xhat if prec == "exact" else float(np.float16(xhat))
            e = sub(x, ref)
            terms.append(abs(e) if metric == "mae" else mul(e, e))
        if nrows == 1:
            err = left_fold(terms) if order == "seq" else lane_tree(terms)
        else:
            err = lane_tree([lane_tree(terms[16 * r:16 * r + 16]) for r in range(16)])
        results[c] = (codes, k, err)
    if recipe == "nvfp4":
        kept = 6
    elif recipe == "map4":
        kept = 4
    else:
        kept = 4 if results[4][2] < results[6][2] else 6
    codes, k, _ = results[kept]
    err6 = results[6][2] if 6 in results else math.nan
    err4 = results[4][2] if 4 in results else math.nan
    return codes, k, kept, err6, err4


def quantize_tensor(x: np.ndarray, amax: np.ndarray, block: str, scale_gran: str, bound: int, recipe: str,
                    metric: str, prec: str, order: str = "tree"):
    """x: float64 array [M, K] of binary32 values. Returns codes [M, K/2],
    scales [M, K/16], kept [nblocks], errs [nblocks, 2]."""
    M, K = x.shape
    nrows = 16 if block == "16x16" else 1
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    kept_l, errs = [], []
    for rb in range(M // nrows):
        r0 = rb * nrows
        A = float(amax[0] if scale_gran == "tensor" else amax[r0])
        for cb in range(K // 16):
            xs = [float(v) for v in x[r0:r0 + nrows, cb * 16:cb * 16 + 16].reshape(-1)]
            q, k, kept, e6, e4 = quantize_block(xs, nrows, A, bound, recipe, metric, prec, order)
            kept_l.append(kept)
            errs.append((e6, e4))
            for i in range(nrows):
                row = q[16 * i:16 * i + 16]
                for j in range(8):
                    codes[r0 + i, cb * 8 + j] = (row[2 * j] & 0xF) | ((row[2 * j + 1] & 0xF) << 4)
                scales[r0 + i, cb] = k
    return codes, scales, np.array(kept_l), np.array(errs, dtype=np.float64)
