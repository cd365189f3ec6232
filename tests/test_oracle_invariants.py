"""Pins: properties of the quantizer that hold whatever the data (CPU only).

Each property is checked on the oracle's outputs with independent numpy
arithmetic: decoded values, candidate errors and the lane-model error tree are
recomputed here from the codes and scales alone.
"""
import numpy as np
import pytest
import torch

import synthdata
from synthdata import raw_bits

OCP_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                    np.float32)
E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()

MODES = [(m, p) for m in ("mae", "mse") for p in ("exact", "fp16")]


def unpack(codes):
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def decode(codes, scales, sdec, gran):
    """x_hat = RN(val(q) * RN(sigma * S_dec)) in numpy float32."""
    q = unpack(codes)
    M, K = q.shape
    sig = np.repeat(E4M3[scales], 16, axis=1)
    s = sdec.reshape(-1, 1) if gran == "row" else sdec.reshape(1, 1)
    D = (sig * s).astype(np.float32)
    return (OCP_E2M1[q] * D).astype(np.float32)


def lane_tree(u):
    """u: [..., 16] float32; clamped shuffle-down by 8, 4, 2, 1, lane 0."""
    lanes = u.astype(np.float32).copy()
    for off in (8, 4, 2, 1):
        src = np.concatenate([lanes[..., off:], lanes[..., 16 - off:]], axis=-1)  # clamped lanes read themselves
        src[..., 16 - off:] = lanes[..., 16 - off:]
        lanes = (lanes + src).astype(np.float32)
    return lanes[..., 0]


def block_errors(x, xhat, metric, prec, block):
    ref = xhat.astype(np.float16).astype(np.float32) if prec == "fp16" else xhat
    with np.errstate(all="ignore"):
        e = (x - ref).astype(np.float32)
        u = np.abs(e) if metric == "mae" else (e * e).astype(np.float32)
    M, K = x.shape
    if block == "1x16":
        return lane_tree(u.reshape(M, K // 16, 16)).reshape(-1)
    t = u.reshape(M // 16, 16, K // 16, 16).transpose(0, 2, 1, 3)  # [band, col-block, row, col]
    rows = lane_tree(t)
    return lane_tree(rows).reshape(-1)


def _x(family, dtype, M, K, seed):
    if family == "weight":
        return synthdata.weight(M, K, seed, dtype)
    return synthdata.activation_family(family, M, K, seed, dtype)


def _values(t):
    return t.to(torch.float32).numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("family", ["normal", "outlier", "special", "weight"])
@pytest.mark.parametrize("block,gran", [("1x16", "tensor"), ("1x16", "row"), ("16x16", "tensor"), ("16x16", "row")])
def test_selection_keeps_lower_recomputed_error(orc, dtype, family, block, gran):
    """Four-over-six output equals, block by block, whichever of the standard
    (map-to-6) and map-to-4-only outputs has the strictly lower error as
    recomputed here from their codes and scales; ties keep map-to-6."""
    M, K = 32, 256
    t = _x(family, dtype, M, K, 101)
    bits, x = raw_bits(t), _values(t)
    mode = "tensor" if gran == "tensor" else ("band16" if block == "16x16" else "row")
    amax = orc.amax(bits, dtype, mode)
    for bound in (448, 256):
        for metric, prec in MODES:
            kw = dict(block=block, scale_gran=gran, err_metric=metric, err_prec=prec, bound=bound)
            r6 = orc.quantize(bits, dtype, amax, recipe="nvfp4", **kw)
            r4 = orc.quantize(bits, dtype, amax, recipe="map4", **kw)
            r = orc.quantize(bits, dtype, amax, recipe="4over6", debug=True, **kw)
            e6 = block_errors(x, decode(r6["codes"], r6["scales"], r6["sdec"], gran), metric, prec, block)
            e4 = block_errors(x, decode(r4["codes"], r4["scales"], r4["sdec"], gran), metric, prec, block)
            np.testing.assert_array_equal(r["err"][:, 0], e6)
            np.testing.assert_array_equal(r["err"][:, 1], e4)
            want = np.where(e4 < e6, 4, 6)
            np.testing.assert_array_equal(r["choice"], want)
            assert np.all(~(e4 < e6) | (e4 <= e6))
            # outputs are the kept candidate's, block by block
            nb_r = K // 16
            ch = want.reshape(M // (16 if block == "16x16" else 1), nb_r)
            if block == "16x16":
                ch = np.repeat(ch, 16, axis=0)
            sc = np.where(ch == 4, r4["scales"], r6["scales"])
            np.testing.assert_array_equal(r["scales"], sc)
            chc = np.repeat(ch, 8, axis=1)
            np.testing.assert_array_equal(r["codes"], np.where(chc == 4, r4["codes"], r6["codes"]))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("k", [-5, 7])
@pytest.mark.parametrize("block", ["1x16", "16x16"])
def test_power_of_two_scale_invariance(orc, dtype, k, block):
    """x * 2^k quantized under amax * 2^k gives identical codes and scales:
    the global scale absorbs the power of two exactly."""
    t = _x("normal", dtype, 32, 128, 7)
    t2 = (t.to(torch.float32) * 2.0 ** k).to(t.dtype)
    b1, b2 = raw_bits(t), raw_bits(t2)
    A = orc.amax(b1, dtype, "tensor") * np.float32(1.3)
    A2 = (A * np.float32(2.0 ** k)).astype(np.float32)
    # (binary16 rounding of the decoded values is not scale-free, so FP16-error mode is left out)
    for recipe in ("nvfp4", "4over6"):
        for metric in ("mae", "mse"):
            kw = dict(recipe=recipe, block=block, err_metric=metric, err_prec="exact")
            r1 = orc.quantize(b1, dtype, A, **kw)
            r2 = orc.quantize(b2, dtype, A2, **kw)
            np.testing.assert_array_equal(r1["codes"], r2["codes"])
            np.testing.assert_array_equal(r1["scales"], r2["scales"])


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_negation_flips_only_sign_bits(orc, dtype):
    t = _x("special", dtype, 32, 128, 9)
    b1, b2 = raw_bits(t), raw_bits(-t)
    A = orc.amax(b1, dtype, "row")
    for metric, prec in MODES:
        kw = dict(recipe="4over6", scale_gran="row", err_metric=metric, err_prec=prec)
        r1 = orc.quantize(b1, dtype, A, **kw)
        r2 = orc.quantize(b2, dtype, A, **kw)
        np.testing.assert_array_equal(r1["scales"], r2["scales"])
        np.testing.assert_array_equal(r1["codes"] ^ 0x88, r2["codes"])


def test_zero_blocks(orc):
    t = synthdata.activation_family("special", 64, 256, 4, "bf16")
    bits, x = raw_bits(t), _values(t)
    A = orc.amax(bits, "bf16", "row")
    r = orc.quantize(bits, "bf16", A, recipe="4over6", scale_gran="row", debug=True)
    zero_blk = (np.abs(x).reshape(64, 16, 16).max(axis=2) == 0).reshape(-1)
    assert zero_blk.sum() > 100
    assert np.all(r["scales"].reshape(-1)[zero_blk] == 0)
    assert np.all(r["choice"][zero_blk] == 6)
    q = unpack(r["codes"]).reshape(-1, 16)[zero_blk]
    sgn = np.signbit(x).reshape(-1, 16)[zero_blk]
    np.testing.assert_array_equal(q, np.where(sgn, 8, 0))
    assert np.all(A[:8] == 0)  # rows 0-7 are all +-0: S_enc = 1 guard
    np.testing.assert_array_equal(r["sdec"][:8], np.ones(8, np.float32))


def test_per_row_with_equal_amax_is_per_tensor(orc):
    t = synthdata.weight(48, 256, 5, "bf16")
    bits = raw_bits(t)
    A = orc.amax(bits, "bf16", "tensor")
    for block in ("1x16", "16x16"):
        r1 = orc.quantize(bits, "bf16", A, recipe="4over6", block=block, scale_gran="tensor")
        r2 = orc.quantize(bits, "bf16", np.full(48, A[0], np.float32), recipe="4over6", block=block,
                          scale_gran="row")
        np.testing.assert_array_equal(r1["codes"], r2["codes"])
        np.testing.assert_array_equal(r1["scales"], r2["scales"])
        assert r2["status"] == 0


def test_16x16_scale_replicated_and_nonuniform_flag(orc):
    t = synthdata.weight(64, 128, 6, "bf16")
    bits = raw_bits(t)
    band = orc.amax(bits, "bf16", "band16")
    r = orc.quantize(bits, "bf16", band, recipe="4over6", block="16x16", scale_gran="row")
    assert r["status"] == 0
    s = r["scales"].reshape(4, 16, 8)
    assert np.all(s == s[:, :1, :])
    row = orc.amax(bits, "bf16", "row")
    r2 = orc.quantize(bits, "bf16", row, recipe="4over6", block="16x16", scale_gran="row")
    assert r2["status"] & 1
    # a non-uniform band is quantized with its first row's amax
    first = np.repeat(row.reshape(4, 16)[:, :1], 16, axis=1).reshape(-1)
    r3 = orc.quantize(bits, "bf16", first, recipe="4over6", block="16x16", scale_gran="row")
    np.testing.assert_array_equal(r2["codes"], r3["codes"])


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_amax_modes(orc, dtype):
    t = synthdata.activation_family("outlier", 64, 96, 8, dtype).to(torch.float32)
    t[3, 5] = float("nan")
    t[17, :] = float("nan")
    t = t.to(synthdata.TORCH_DTYPES[dtype])
    x = np.abs(_values(t))
    x = np.where(np.isnan(x), 0, x)
    bits = raw_bits(t)
    assert orc.amax(bits, dtype, "tensor")[0] == x.max()
    np.testing.assert_array_equal(orc.amax(bits, dtype, "row"), x.max(axis=1))
    np.testing.assert_array_equal(orc.amax(bits, dtype, "band16"), np.repeat(x.reshape(4, 16, 96).max(axis=(1, 2)), 16))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("recipe,metric,prec", [("nvfp4", "mse", "exact")] + [("4over6", m, p) for m, p in MODES])
@pytest.mark.parametrize("bound", [448, 256])
def test_qdq_is_dequantize_of_quantize(orc, dtype, recipe, metric, prec, bound):
    t = synthdata.activation_family("outlier", 32, 256, 12, dtype)
    bits = raw_bits(t)
    A = orc.amax(bits, dtype, "tensor")
    kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound)
    q = orc.quantize(bits, dtype, A, **kw)
    y = orc.qdq(bits, dtype, A, **kw)
    y2 = orc.dequantize(q["codes"], q["scales"], q["sdec"], "tensor", dtype)
    np.testing.assert_array_equal(y, y2)
    # and the dequantized values are the numpy recomputation rounded to the dtype
    xh = decode(q["codes"], q["scales"], q["sdec"], "tensor")
    want = raw_bits(torch.from_numpy(xh).to(synthdata.TORCH_DTYPES[dtype]))
    np.testing.assert_array_equal(y, want)


def _round_to(xh: np.ndarray, dtype: str) -> np.ndarray:
    """Raw bits of float32 values rounded to dtype (RNE, overflow to inf) by
    numpy (fp16) or torch (bf16), independently of the oracle's rounding."""
    if dtype == "fp32":
        return xh.astype(np.float32)
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return xh.astype(np.float16).view(np.uint16)
    return raw_bits(torch.from_numpy(xh).to(torch.bfloat16))


def _cmp_bits(a, b, msg=""):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    np.testing.assert_array_equal(a, b, err_msg=msg)


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("gran", ["tensor", "row"])
def test_dequantize_matches_independent_decode(orc, out_dtype, gran):
    """nvfp4_dequantize (pytorch/ao PR, recipe commit: the recipe-agnostic
    decode, with row-scaled global scales) on random codes covering all 16
    nibbles, random finite block scales and S_dec that differs from row to
    row (a wide range: fp16 outputs overflow to inf, some underflow), equals
    the numpy decode RN(val(q) * RN(sigma * S_dec)) rounded to the output
    type by numpy or torch."""
    M, K = 48, 160
    codes = synthdata.random_packed_codes(M, K, 91)
    scales = synthdata.random_block_scales(M, K, 92)
    rng = np.random.default_rng(93)
    n = M if gran == "row" else 1
    sdec = (2.0 ** rng.uniform(-30, 12, n)).astype(np.float32)
    if gran == "row":
        sdec[:4] = [1.0, 2.0 ** -140, 3.0e-3, 7.5]  # includes a subnormal S_dec
    y = orc.dequantize(codes, scales, sdec, gran, out_dtype)
    _cmp_bits(y, _round_to(decode(codes, scales, sdec, gran), out_dtype), f"{out_dtype} {gran}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("block,gran", [("1x16", "tensor"), ("1x16", "row"), ("16x16", "tensor"), ("16x16", "row")])
def test_qdq_every_dtype_block_and_granularity(orc, dtype, block, gran):
    """The fused QDQ output is the kept candidate's decoded values rounded
    once to the input type, for every input type, block shape and scale
    granularity the quantizer takes: it equals the numpy decode of the
    quantizer's own codes, scales and S_dec, rounded by numpy or torch. The
    16x16 per-row amax is uniform within each band (the tile-uniform
    contract), and the per-row S_dec differs from band to band."""
    M, K = 64, 192
    t = _x("outlier", dtype, M, K, 111)
    bits = raw_bits(t)
    mode = "tensor" if gran == "tensor" else ("band16" if block == "16x16" else "row")
    amax = orc.amax(bits, dtype, mode)
    for (recipe, metric, prec), bound in [(("nvfp4", "mse", "exact"), 448), (("4over6", "mse", "exact"), 448),
                                          (("4over6", "mae", "fp16"), 256)]:
        kw = dict(recipe=recipe, block=block, scale_gran=gran, err_metric=metric, err_prec=prec, bound=bound)
        q = orc.quantize(bits, dtype, amax, **kw)
        y = orc.qdq(bits, dtype, amax, **kw)
        _cmp_bits(y, _round_to(decode(q["codes"], q["scales"], q["sdec"], gran), dtype), f"{dtype} {kw}")


def test_grouped_equals_per_group(orc):
    M, pad, K, G = 512, 48, 128, 12
    x, offs, fac = synthdata.grouped_tokens(M, pad, K, G, seeds=(1, 2, 3, 4))
    bits = raw_bits(x)
    starts = np.concatenate([[0], offs[:-1]])
    gam = np.array([orc.amax(bits[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    for bound in (448, 256):
        r = orc.quantize_grouped(bits, "bf16", offs, gam, recipe="4over6", bound=bound)
        assert r["status"] == 0
        for g in range(G):
            s, e = starts[g], offs[g]
            if e == s:
                continue
            rg = orc.quantize(bits[s:e], "bf16", gam[g:g + 1], recipe="4over6", bound=bound)
            np.testing.assert_array_equal(r["codes"][s:e], rg["codes"])
            np.testing.assert_array_equal(r["scales"][s:e], rg["scales"])
            assert r["group_sdec"][g] == rg["sdec"][0]
        assert np.all(r["codes"][M:] == 0) and np.all(r["scales"][M:] == 0)


def test_grouped_empty_groups_and_bad_offsets(orc):
    K = 64
    x = raw_bits(synthdata.normal(96, K, 3, "bf16"))
    offs = np.array([0, 32, 32, 64, 64], np.int32)  # empty groups 0, 2 and 4
    gam = np.array([5.0, 2.0, 7.0, 3.0, 9.0], np.float32)
    r = orc.quantize_grouped(x, "bf16", offs, gam, recipe="4over6")
    r1 = orc.quantize(x[:32], "bf16", gam[1:2], recipe="4over6")
    r3 = orc.quantize(x[32:64], "bf16", gam[3:4], recipe="4over6")
    np.testing.assert_array_equal(r["codes"][:32], r1["codes"])
    np.testing.assert_array_equal(r["codes"][32:64], r3["codes"])
    assert np.all(r["codes"][64:] == 0)
    for bad in ([0, 40, 32, 64, 64], [0, 33, 48, 64, 64], [0, 32, 48, 64, 112]):
        rb = orc.quantize_grouped(x, "bf16", np.array(bad, np.int32), gam, recipe="4over6")
        assert rb["status"] & 2
