"""Admissibility of the gfx950 converts and of the FMA-corrected division by
6: the kernels' own device helpers (fos_device.h, compiled with the
library's flags into tests/libfos_primitives.so) run on the GPU over every
input the kernels can feed them, and each result is compared bitwise with
the CPU: the oracle's E2M1, E4M3, binary16 and bfloat16 conversions and
global scales, and IEEE binary32 division, subtraction and multiplication
as numpy computes them. The first mismatch fails the test.

The wolfcomos/ao PR "Add a CuTe DSL fast-path kernel for four-over-six
quantize" (description) names these rounding-critical steps: correctly
rounded FP32 division, the FP4 (E2M1) and E4M3 casts, and their decodes.

Input domains (what the kernels can feed each helper):
  - E2M1 encode: any binary32 (x * E, NaN included): every 2^32 pattern.
  - E4M3 encode: t = RN(q * S_enc) >= 0, never NaN: every pattern from +0
    to +inf.
  - division by 6: the block amax a >= 0 (NaN dropped): +0 .. +inf.
  - global scales: the amax A, any pattern (caller-supplied amaxes can be
    negative or NaN): every 2^32 pattern.
  - bf16 / f16 output rounding: any binary32: every 2^32 pattern.
  - E2M1 decode: every code in every nibble position; E4M3 decode: all 256.
  - FP16-error difference x - f32(RN16(xh)): every (x, xh) pair for 16-bit
    inputs (2^32 pairs per input type), a sample for fp32 inputs.
  - the per-block multiplier table S_enc / sigma and sigma * S_dec: every
    E4M3 sigma against a sample of S_enc.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfos_primitives.so")
SRC = os.path.join(HERE, "gpu_primitives.hip")
CHUNK = 1 << 28  # inputs per launch

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SIGS = {
    "prim_e2m1_encode": [_U32, _I64, _P, _P],
    "prim_e2m1_decode": [_P, _I64, _P, _P],
    "prim_e4m3_encode": [_U32, _I64, _P, _P, _P],
    "prim_e4m3_decode": [_P, _P],
    "prim_div6": [_U32, _I64, _P, _P],
    "prim_global_scales": [_U32, _I64, ctypes.c_float, _P, _P, _P],
    "prim_div_mul": [_P, _P, _I64, _P, _P, _P],
    "prim_pack16": [_I, _U32, _I64, _P, _P, _P],
    "prim_upcast16": [_I, _P, _P],
    "prim_sub_f16_pairs": [_I, _U32, _I64, _P, _P, _P],
    "prim_sub_f16": [_P, _P, _I64, _P, _P, _P],
}


@pytest.fixture(scope="module")
def prim():
    if not os.path.exists(LIB_PATH):
        from nvfp4_adaptive_block_amd import build as fos_build
        fos_build.build(out=LIB_PATH, sources=[SRC])
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        getattr(lib, name).restype = _I
        getattr(lib, name).argtypes = args
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Host:
    """A pinned host buffer per shape/dtype, reused across chunks."""

    def __init__(self):
        self.bufs = {}

    def get(self, t: torch.Tensor) -> np.ndarray:
        key = (t.dtype, t.numel())
        if key not in self.bufs:
            self.bufs[key] = torch.empty(t.numel(), dtype=t.dtype, pin_memory=True)
        h = self.bufs[key]
        h.copy_(t.reshape(-1), non_blocking=True)
        torch.cuda.synchronize()
        return h.numpy()


def _patterns(base: int, n: int) -> np.ndarray:
    return np.arange(base, base + n, dtype=np.uint32)


def _first_mismatch(got_bits, want_bits, inputs, what):
    bad = np.flatnonzero(got_bits != want_bits)
    if bad.size:
        i = bad[0]
        pytest.fail(f"{what}: {bad.size} mismatches; first at input 0x{int(inputs[i]):08x}: "
                    f"got 0x{int(got_bits[i]):x}, want 0x{int(want_bits[i]):x}")


def _is_nan16(bits: np.ndarray, f16: bool) -> np.ndarray:
    exp = 0x7C00 if f16 else 0x7F80
    man = 0x03FF if f16 else 0x007F
    return ((bits & exp) == exp) & ((bits & man) != 0)


# ------------------------------------------------------------------ E2M1

def test_e2m1_encode_every_binary32(prim, orc):
    """v_cvt_scalef32_pk_fp4_f32 with scale 1 is the oracle's RNE-saturating
    E2M1 cast on every non-NaN binary32; a NaN gives (sign | 7), which the
    kernels never store (their careful form encodes NaN as +6 first)."""
    out = torch.empty(CHUNK // 8, dtype=torch.int32, device="cuda")
    host = Host()
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, :]
    for base in range(0, 1 << 32, CHUNK):
        assert prim.prim_e2m1_encode(base, CHUNK // 8, _p(out), _s()) == 0
        words = host.get(out).view(np.uint32)
        got = ((words[:, None] >> shifts) & 0xF).astype(np.uint8).reshape(-1)
        x = _patterns(base, CHUNK)
        want = orc.e2m1_rne_sat(x.view(np.float32))
        nan = (x & 0x7FFFFFFF) > 0x7F800000
        want = np.where(nan, (7 | ((x >> 31) << 3)).astype(np.uint8), want)
        _first_mismatch(got, want, x, "E2M1 encode")


def test_e2m1_decode_every_code_in_every_position(prim, orc):
    """v_cvt_scalef32_pk_f32_fp4 with scale 1 decodes every code exactly,
    signed zero included, in each of the eight nibble positions."""
    codes = np.arange(16, dtype=np.uint32)
    words = [(codes << (4 * k)) for k in range(8)]
    words.append(np.random.default_rng(5).integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32))
    words = np.concatenate(words)
    w = torch.from_numpy(words.view(np.int32)).to("cuda")
    out = torch.empty(words.size * 8, dtype=torch.float32, device="cuda")
    assert prim.prim_e2m1_decode(_p(w), words.size, _p(out), _s()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(-1, 8)
    table = np.array([orc.e2m1_value(c) for c in range(16)], np.float32).view(np.uint32)
    want = table[(words[:, None] >> (4 * np.arange(8, dtype=np.uint32))[None, :]) & 0xF]
    _first_mismatch(got.reshape(-1), want.reshape(-1), np.repeat(words, 8), "E2M1 decode")


# ------------------------------------------------------------------ E4M3

def test_e4m3_encode_every_nonnegative_input(prim, orc):
    """min(t, 448) then v_cvt_pk_fp8_f32 is the oracle's RNE-saturating E4M3
    cast for every t from +0 to +inf, and the word's upper bytes are zero."""
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    upper = torch.zeros(1, dtype=torch.int32, device="cuda")
    host = Host()
    end = 0x7F800001
    for base in range(0, end, CHUNK):
        n = min(CHUNK, end - base)
        assert prim.prim_e4m3_encode(base, n, _p(out), _p(upper), _s()) == 0
        got = host.get(out)[:n]
        t = _patterns(base, n)
        _first_mismatch(got, orc.e4m3_rne_sat(t.view(np.float32)), t, "E4M3 encode")
    assert int(upper.item()) == 0, "the convert's upper bytes are not zero"


def test_e4m3_decode_every_code(prim, orc):
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    assert prim.prim_e4m3_decode(_p(out), _s()) == 0
    got = out.cpu().numpy()
    want = np.array([orc.e4m3_value(c) for c in range(256)], np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


# ------------------------------------------------------------------ division and global scales

def test_div6_every_nonnegative_input(prim):
    """div6(a), the FMA-corrected product with RN(1/6) (true division below
    2^-125), is IEEE RN(a / 6) for every a from +0 to +inf."""
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    host = Host()
    end = 0x7F800001
    six = np.float32(6.0)
    for base in range(0, end, CHUNK):
        n = min(CHUNK, end - base)
        assert prim.prim_div6(base, n, _p(out), _s()) == 0
        got = host.get(out)[:n].view(np.uint32)
        a = _patterns(base, n)
        want = (a.view(np.float32) / six).view(np.uint32)
        _first_mismatch(got, want, a, "RN(a / 6)")


@pytest.mark.parametrize("bound", [448, 256])
def test_global_scales_every_amax(prim, orc, bound):
    """S_enc = min(RN(6B / A), FLT_MAX) (1 when A is not in (0, inf)) and
    S_dec = RN(1 / S_enc) on the device equal the oracle's for every binary32
    amax pattern (caller-supplied amaxes can be negative or NaN)."""
    enc = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    dec = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    he, hd = Host(), Host()
    for base in range(0, 1 << 32, CHUNK):
        assert prim.prim_global_scales(base, CHUNK, 6.0 * bound, _p(enc), _p(dec), _s()) == 0
        ge, gd = he.get(enc).view(np.uint32), hd.get(dec).view(np.uint32)
        A = _patterns(base, CHUNK)
        we, wd = orc.global_scales(A.view(np.float32), bound)
        _first_mismatch(ge, we.view(np.uint32), A, f"S_enc (bound {bound})")
        _first_mismatch(gd, wd.view(np.uint32), A, f"S_dec (bound {bound})")


def test_multiplier_table_division_and_products(prim):
    """The per-block multipliers RN(S_enc / sigma) and RN(sigma * S_dec) for
    every non-zero E4M3 sigma and a sample of S_enc (log-uniform over the
    whole binary32 range, plus FLT_MAX and subnormals) are IEEE binary32
    quotients and products."""
    rng = np.random.default_rng(7)
    s = (2.0 ** rng.uniform(-149, 128, 1 << 17)).astype(np.float32)
    s = np.concatenate([s, np.array([np.finfo(np.float32).max, 1e-45, 1e-40, 1.0, 6.0], np.float32)])
    s = s[np.isfinite(s) & (s > 0)]
    sig = torch.arange(1, 127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    a = np.repeat(s, sig.size)
    b = np.tile(sig, s.size)
    ad, bd = torch.from_numpy(a).to("cuda"), torch.from_numpy(b).to("cuda")
    q = torch.empty_like(ad)
    p = torch.empty_like(ad)
    assert prim.prim_div_mul(_p(ad), _p(bd), a.size, _p(q), _p(p), _s()) == 0
    torch.cuda.synchronize()
    with np.errstate(over="ignore", under="ignore"):
        _first_mismatch(q.cpu().numpy().view(np.uint32), (a / b).view(np.uint32), a.view(np.uint32), "S_enc / sigma")
        _first_mismatch(p.cpu().numpy().view(np.uint32), (a * b).view(np.uint32), a.view(np.uint32), "sigma * S_dec")


# ------------------------------------------------------------------ 16-bit conversions

@pytest.mark.parametrize("f16", [0, 1], ids=["bf16", "f16"])
def test_output_rounding_every_binary32(prim, orc, f16):
    """pack_bf16 / pack_f16 (one packed convert: the QDQ and dequantize
    outputs, and the binary16 rounding of the FP16-error mode) round every
    binary32 as the oracle does (RNE, overflow to inf, gradual underflow),
    in the low half and, swapped, in the high half; a NaN input gives a
    NaN."""
    out = torch.empty(CHUNK // 2, dtype=torch.int32, device="cuda")
    mismatch = torch.zeros(1, dtype=torch.int32, device="cuda")
    host = Host()
    conv = orc.f32_to_f16_bits if f16 else orc.f32_to_bf16_bits
    for base in range(0, 1 << 32, CHUNK):
        assert prim.prim_pack16(f16, base, CHUNK // 2, _p(out), _p(mismatch), _s()) == 0
        got = host.get(out).view(np.uint16)  # little-endian: element 2t, then 2t + 1
        x = _patterns(base, CHUNK)
        want = conv(x.view(np.float32))
        nan_in = (x & 0x7FFFFFFF) > 0x7F800000
        assert np.all(_is_nan16(got[nan_in], f16)), "a NaN input did not give a NaN"
        _first_mismatch(np.where(nan_in, 0, got), np.where(nan_in, 0, want), x,
                        "f16 rounding" if f16 else "bf16 rounding")
    assert int(mismatch.item()) == 0, "a value rounds differently in the low and the high half"


@pytest.mark.parametrize("f16", [0, 1], ids=["bf16", "f16"])
def test_input_upcasts_every_16bit_pattern(prim, f16):
    out = torch.empty(65536, dtype=torch.float32, device="cuda")
    assert prim.prim_upcast16(f16, _p(out), _s()) == 0
    got = out.cpu().numpy()
    h = np.arange(65536, dtype=np.uint32)
    if f16:
        want = h.astype(np.uint16).view(np.float16).astype(np.float32)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    else:
        np.testing.assert_array_equal(got.view(np.uint32), h << 16)


# ------------------------------------------------------------------ FP16-error difference

@pytest.mark.parametrize("x_f16", [0, 1], ids=["bf16_x", "f16_x"])
def test_fp16_error_difference_every_16bit_pair(prim, x_f16):
    """sub_f16x2 (a packed binary16 convert, then per element one
    v_fma_mix_f32: the binary16 operand times -1, plus x, rounded once)
    equals IEEE RN(x - f32(h)) for every x of the 16-bit input type and
    every binary16 h, in the low and in the high half; NaN results agree as
    NaN."""
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    mismatch = torch.zeros(1, dtype=torch.int32, device="cuda")
    host = Host()
    h_val = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    rows = CHUNK >> 16
    for base in range(0, 1 << 32, CHUNK):
        assert prim.prim_sub_f16_pairs(x_f16, base, CHUNK, _p(out), _p(mismatch), _s()) == 0
        got = host.get(out).reshape(rows, 65536)
        xw = np.arange(base >> 16, (base >> 16) + rows, dtype=np.uint32)
        x = xw.astype(np.uint16).view(np.float16).astype(np.float32) if x_f16 else (xw << 16).view(np.float32)
        with np.errstate(invalid="ignore", over="ignore"):
            want = (x[:, None] - h_val[None, :]).astype(np.float32)
        gn, wn = np.isnan(got), np.isnan(want)
        assert np.array_equal(gn, wn), "NaN results differ"
        g = np.where(gn, 0, got).view(np.uint32).reshape(-1)
        w = np.where(wn, 0, want).view(np.uint32).reshape(-1)
        _first_mismatch(g, w, _patterns(base, CHUNK), "x - f32(h)")
    assert int(mismatch.item()) == 0, "a difference depends on the half it is computed in"


def test_fp16_error_difference_fp32_operands(prim, orc):
    """For fp32 inputs (x any binary32) and decoded values that are not
    binary16 values, sub_f16x2 gives RN(x - f32(RN16(xh))) in either half, on
    a sample that covers every binade, subnormals, overflow to inf and NaN."""
    rng = np.random.default_rng(11)
    n = 1 << 24
    x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    xh = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    # half the pairs near each other (small differences, cancellation)
    near = rng.random(n) < 0.5
    xh[near] = (x[near].astype(np.int64) + rng.integers(-(1 << 14), 1 << 14, int(near.sum()))).astype(np.uint32)
    xd = torch.from_numpy(x.view(np.float32)).to("cuda")
    hd = torch.from_numpy(xh.view(np.float32)).to("cuda")
    out = torch.empty_like(xd)
    mismatch = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert prim.prim_sub_f16(_p(xd), _p(hd), n, _p(out), _p(mismatch), _s()) == 0
    torch.cuda.synchronize()
    assert int(mismatch.item()) == 0, "a difference depends on the half it is computed in"
    got = out.cpu().numpy()
    h = orc.f32_to_f16_bits(xh.view(np.float32)).view(np.float16).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        want = (x.view(np.float32) - h).astype(np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), "NaN results differ"
    _first_mismatch(np.where(gn, 0, got).view(np.uint32), np.where(wn, 0, want).view(np.uint32), x, "x - f32(RN16(xh))")
