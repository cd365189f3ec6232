"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Every case feeds the same seeded input bits to both sides; amaxes and group
offsets come from the oracle or the input generators, never from the GPU.
Codes, scales and S_dec must match exactly; dequantized and QDQ outputs are
compared as raw 16-bit patterns (signed zeros included).
"""
import itertools

import numpy as np
import pytest
import torch

import nvfp4_adaptive_block_amd as fos
import synthdata
from synthdata import raw_bits

pytestmark = pytest.mark.gpu

MODES = [("nvfp4", "mse", "exact")] + [("4over6", m, p) for m in ("mae", "mse") for p in ("exact", "fp16")]


def dev(t):
    return t.to("cuda")


def u_bits(a: np.ndarray) -> np.ndarray:
    """Integer view of raw element bits (fp32 arrays as uint32), so that
    comparisons are bitwise: signed zeros and NaN payloads included."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def bits_of(t: torch.Tensor) -> np.ndarray:
    return raw_bits(t.cpu())


def gpu_quant(x, amax, **kw):
    codes, scales, sdec = fos.fos_quantize(dev(x), dev(torch.from_numpy(amax)), **kw)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), sdec.cpu().numpy()


def assert_quant_equal(orc, x, dtype, amax, label="", **kw):
    want = orc.quantize(raw_bits(x), dtype, amax, **kw)
    codes, scales, sdec = gpu_quant(x, amax, **kw)
    np.testing.assert_array_equal(scales, want["scales"], err_msg=f"scales {label} {kw}")
    np.testing.assert_array_equal(codes, want["codes"], err_msg=f"codes {label} {kw}")
    np.testing.assert_array_equal(sdec.view(np.uint32), want["sdec"].view(np.uint32), err_msg=f"sdec {label} {kw}")


def _family(family, dtype, M, K, seed):
    if family == "weight":
        return synthdata.weight(M, K, seed, dtype)
    return synthdata.activation_family(family, M, K, seed, dtype)


# ------------------------------------------------------------------ 1x16

def test_single_tensor_256x1024(orc):
    """bf16 256x1024 N(0,1), per-tensor amax, 1x16, bound 448, MSE exact; then every mode."""
    x = synthdata.normal(256, 1024, 11, "bf16")
    amax = orc.amax(raw_bits(x), "bf16", "tensor")
    assert_quant_equal(orc, x, "bf16", amax, recipe="4over6", err_metric="mse", err_prec="exact", bound=448)
    for (recipe, metric, prec), bound, gran in itertools.product(MODES, (448, 256), ("tensor", "row")):
        a = amax if gran == "tensor" else orc.amax(raw_bits(x), "bf16", "row")
        assert_quant_equal(orc, x, "bf16", a, recipe=recipe, err_metric=metric, err_prec=prec, bound=bound,
                           scale_gran=gran)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("family", synthdata.ACTIVATION_FAMILIES)
def test_activation_families_all_knobs(orc, dtype, family):
    """The dense-activation families at a size with ragged rows (K/16 = 97
    blocks per row, units straddle rows), both global-scale granularities,
    every mode and both bounds."""
    M, K = 67, 1552
    x = _family(family, dtype, M, K, 21 + synthdata.ACTIVATION_FAMILIES.index(family))
    b = raw_bits(x)
    am = {"tensor": orc.amax(b, dtype, "tensor"), "row": orc.amax(b, dtype, "row")}
    for (recipe, metric, prec), bound, gran in itertools.product(MODES, (448, 256), ("tensor", "row")):
        assert_quant_equal(orc, x, dtype, am[gran], label=family, recipe=recipe, err_metric=metric, err_prec=prec,
                           bound=bound, scale_gran=gran)


@pytest.mark.parametrize("shape", [(1, 16), (1, 1024), (3, 48), (5, 1008), (130, 64), (2, 2064)])
def test_small_and_ragged_shapes(orc, shape):
    M, K = shape
    x = synthdata.activation_family("outlier", M, K, 5, "bf16")
    b = raw_bits(x)
    for gran in ("tensor", "row"):
        a = orc.amax(b, "bf16", gran)
        for recipe, metric, prec in MODES:
            assert_quant_equal(orc, x, "bf16", a, recipe=recipe, err_metric=metric, err_prec=prec, scale_gran=gran)


def test_caller_amax_edge_values(orc):
    """Caller amax below the data (scales saturate), zero, inf, NaN, tiny
    (S_enc clamps to FLT_MAX) and huge."""
    x = synthdata.activation_family("normal", 32, 256, 6, "fp32")
    b = raw_bits(x)
    true = float(orc.amax(b, "fp32", "tensor")[0])
    for A in (true / 7, 0.0, float("inf"), float("nan"), 1e-38, 1e-45, 3e38, -1.0):
        a = np.array([A], np.float32)
        for recipe, metric, prec in MODES:
            assert_quant_equal(orc, x, "fp32", a, label=f"A={A}", recipe=recipe, err_metric=metric, err_prec=prec)



def test_fp16_error_mode_past_binary16_range(orc):
    """FP16-error mode where decoded values leave binary16's range: blocks of
    magnitudes around and past 65504 (x-hat rounds to inf in binary16, so a
    candidate's error terms turn infinite or NaN), blocks below its subnormal
    range (x-hat rounds to zero or a subnormal), and ordinary blocks with one
    huge element; the quantize with per-tensor and per-row scales and the
    QDQ, bf16 and fp32 inputs, against the oracle."""
    rng = np.random.default_rng(71)
    M, K = 48, 272
    x = np.empty((M, K))
    x[:16] = rng.uniform(3.0e4, 2.0e5, (16, K))
    x[16:32] = 10.0 ** rng.uniform(-10, -6, (16, K))
    x[32:] = rng.standard_normal((16, K))
    x[32:, ::16] = 1.0e5
    x = (x * np.where(rng.random((M, K)) < 0.5, -1.0, 1.0)).astype(np.float32)
    for dtype in ("fp32", "bf16"):
        xt = torch.from_numpy(x).to(synthdata.TORCH_DTYPES[dtype])
        b = raw_bits(xt)
        for gran in ("tensor", "row"):
            a = orc.amax(b, dtype, gran)
            for metric in ("mae", "mse"):
                assert_quant_equal(orc, xt, dtype, a, label=f"{dtype} {gran}", recipe="4over6", err_metric=metric,
                                   err_prec="fp16", scale_gran=gran)
        a = orc.amax(b, dtype, "tensor")
        for metric in ("mae", "mse"):
            y = fos.fos_qdq(dev(xt), dev(torch.from_numpy(a)), recipe="4over6", err_metric=metric, err_prec="fp16")
            torch.cuda.synchronize()
            want = orc.qdq(b, dtype, a, recipe="4over6", err_metric=metric, err_prec="fp16")
            np.testing.assert_array_equal(u_bits(bits_of(y)), u_bits(want), err_msg=f"qdq {dtype} {metric}")

def test_nan_inf_and_signed_zero_blocks(orc):
    """NaN (quiet and signalling, both signs), +-inf, +-0, subnormals: the
    careful path and the NaN rule (+6)."""
    M, K = 16, 64
    x = np.random.default_rng(3).standard_normal((M, K)).astype(np.float32)
    u = x.view(np.uint32)
    u[0, 0] = 0x7FC00000   # qNaN
    u[1, 5] = 0xFFC00001   # -qNaN
    u[2, 7] = 0x7F800001   # sNaN
    u[3, 3] = 0xFF800005   # -sNaN
    u[3, 4] = 0x7F800001
    x[4, :16] = np.inf
    x[5, 3] = -np.inf
    x[6, :16] = -0.0
    x[7, :16] = 0.0
    x[7, 5] = -0.0
    x[8, :] = 1e-42
    u[9, :16] = 0x7FC00000  # an all-NaN block: amax +0
    u[10, 16:32] = 0xFF800001
    x[10, 20] = 2.5
    xt = torch.from_numpy(x)
    for dtype in ("fp32", "bf16", "fp16"):
        t = xt.to(synthdata.TORCH_DTYPES[dtype])
        b = raw_bits(t)
        for gran in ("tensor", "row"):
            a = orc.amax(b, dtype, gran)
            for recipe, metric, prec in MODES:
                assert_quant_equal(orc, t, dtype, a, label=dtype, recipe=recipe, err_metric=metric, err_prec=prec,
                                   scale_gran=gran)


# ------------------------------------------------------------------ 16x16

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_16x16_all_knobs(orc, dtype):
    """16x16 tiles on weights, 17 tiles per band (the last group of four
    tiles is ragged), per-tensor and tile-uniform per-row amax."""
    M, K = 48, 272
    x = synthdata.weight(M, K, 31, dtype)
    b = raw_bits(x)
    am = {"tensor": orc.amax(b, dtype, "tensor"), "row": orc.amax(b, dtype, "band16")}
    for (recipe, metric, prec), bound, gran in itertools.product(MODES, (448, 256), ("tensor", "row")):
        assert_quant_equal(orc, x, dtype, am[gran], recipe=recipe, err_metric=metric, err_prec=prec, bound=bound,
                           scale_gran=gran, block="16x16")


def test_16x16_special_data_and_nonuniform_flag(orc):
    M, K = 32, 128
    x = synthdata.activation_family("special", M, K, 8, "bf16").to(torch.float32)
    x[20, 3] = float("nan")
    x[17, 40] = float("inf")
    x = x.to(torch.bfloat16)
    b = raw_bits(x)
    row = orc.amax(b, "bf16", "row")   # not uniform within bands
    for recipe, metric, prec in MODES:
        want = orc.quantize(b, "bf16", row, recipe=recipe, err_metric=metric, err_prec=prec, block="16x16",
                            scale_gran="row")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        codes, scales, sdec = fos.fos_quantize(dev(x), dev(torch.from_numpy(row)), recipe=recipe, err_metric=metric,
                                               err_prec=prec, block="16x16", scale_gran="row", status=status)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
        assert want["status"] & fos.STATUS_TILE_NONUNIFORM
        assert int(status.item()) & fos.STATUS_TILE_NONUNIFORM


@pytest.mark.parametrize("dtype,M,K,out", [("bf16", 4096, 16384, "quantize"), ("fp32", 2048, 16384, "quantize"),
                                            ("bf16", 4096, 8192, "qdq")])
def test_16x16_careful_tiles_between_prefetched_units(orc, dtype, M, K, out):
    """Tiles that need the careful form (a NaN or an inf) scattered over a
    tensor large enough that every wave takes several units: a tile whose
    fast form fails reloads its rows after the next unit's rows were already
    requested in their place, then requests them again. Every output must
    still match the oracle (whole tensors compared)."""
    w = synthdata.weight(M, K, 33, dtype).to(torch.float32)
    a = orc.amax(raw_bits(w.to(synthdata.TORCH_DTYPES[dtype])), dtype, "tensor")  # of the finite data
    g = torch.Generator().manual_seed(34)
    ntiles = (M // 16) * (K // 16)
    tiles = torch.randperm(ntiles, generator=g)[: ntiles // 200]
    r0 = (tiles // (K // 16)) * 16 + torch.randint(0, 16, tiles.shape, generator=g)
    c0 = (tiles % (K // 16)) * 16 + torch.randint(0, 16, tiles.shape, generator=g)
    half = tiles.numel() // 2
    w[r0[:half], c0[:half]] = float("nan")
    w[r0[half:], c0[half:]] = float("inf")
    w[0:16, 0:16] = float("nan")  # one all-NaN tile
    x = w.to(synthdata.TORCH_DTYPES[dtype])
    b = raw_bits(x)
    xd, ad = dev(x), dev(torch.from_numpy(a))
    modes = [("4over6", "mse", "exact"), ("4over6", "mae", "fp16"), ("nvfp4", "mse", "exact")]
    for recipe, metric, prec in modes:
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, block="16x16")
        if out == "quantize":
            want = orc.quantize(b, dtype, a, **kw)
            codes, scales, _ = fos.fos_quantize(xd, ad, **kw)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"scales {kw}")
            np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"codes {kw}")
        else:
            want = orc.qdq(b, dtype, a, **kw)
            y = fos.fos_qdq(xd, ad, **kw)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(bits_of(y), want, err_msg=f"qdq {kw}")


# ------------------------------------------------------------------ QDQ and dequantize

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_qdq_list_all_modes(orc, dtype):
    """A list of expert-like weights of different shapes in one call; each
    output bit-equal to the oracle's fused QDQ."""
    shapes = [(48, 112), (16, 1024), (33, 2064), (1, 16)]
    ws = []
    for i, (M, K) in enumerate(shapes):
        w = torch.randn(M, K, generator=torch.Generator().manual_seed(100 + i)) * 0.02
        w.view(-1)[:: 97] *= 50
        ws.append(w.to(synthdata.TORCH_DTYPES[dtype]))
    amaxes = [orc.amax(raw_bits(w), dtype, "tensor") for w in ws]
    for (recipe, metric, prec), bound in itertools.product(MODES, (448, 256)):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound)
        ys = fos.fos_qdq_list([dev(w) for w in ws], [dev(torch.from_numpy(a)) for a in amaxes], **kw)
        torch.cuda.synchronize()
        for w, a, y in zip(ws, amaxes, ys):
            want = orc.qdq(raw_bits(w), dtype, a, **kw)
            np.testing.assert_array_equal(bits_of(y), want, err_msg=f"{kw} {tuple(w.shape)}")


def test_qdq_single_and_many_tensors(orc):
    """fos_qdq, and a list longer than one launch holds (two launches)."""
    ws = [synthdata.weight(16, 64 + 16 * (i % 5), 200 + i, "bf16") for i in range(53)]
    amaxes = [orc.amax(raw_bits(w), "bf16", "tensor") for w in ws]
    ys = fos.fos_qdq_list([dev(w) for w in ws], [dev(torch.from_numpy(a)) for a in amaxes], recipe="4over6")
    y0 = fos.fos_qdq(dev(ws[0]), dev(torch.from_numpy(amaxes[0])), recipe="4over6")
    torch.cuda.synchronize()
    for w, a, y in zip(ws, amaxes, ys):
        np.testing.assert_array_equal(bits_of(y), orc.qdq(raw_bits(w), "bf16", a, recipe="4over6"))
    np.testing.assert_array_equal(bits_of(y0), bits_of(ys[0]))


@pytest.mark.parametrize("n", [2, 16, 17])
def test_qdq_list_table_limit(orc, n):
    """Lists of up to 16 tensors take the launch's units round robin with a
    table per tensor in LDS; 17 take contiguous ranges. Both sides of the
    limit, with ragged shapes, an empty tensor and tensors smaller than a
    unit, for the plain and the fused-amax list."""
    shapes = [(16 + 16 * (i % 4), 16 * (1 + (7 * i) % 23)) for i in range(n)]
    shapes[n // 2] = (0, 48)
    ws = [synthdata.weight(max(M, 1), K, 500 + i, "fp16")[:M].contiguous() for i, (M, K) in enumerate(shapes)]
    amaxes = [orc.amax(raw_bits(w), "fp16", "tensor") if w.numel() else np.zeros(1, np.float32) for w in ws]
    kw = dict(recipe="4over6", err_metric="mae", err_prec="exact", bound=256)
    ys = fos.fos_qdq_list([dev(w) for w in ws], [dev(torch.from_numpy(a)) for a in amaxes], **kw)
    ysf, amf = fos.fos_qdq_list_fused([dev(w) for w in ws], **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(amf.cpu().numpy().view(np.uint32), np.concatenate(amaxes).view(np.uint32))
    for i, (w, a) in enumerate(zip(ws, amaxes)):
        if w.numel():
            want = orc.qdq(raw_bits(w), "fp16", a, **kw)
            np.testing.assert_array_equal(bits_of(ys[i]), want, err_msg=f"tensor {i} of {n}")
            np.testing.assert_array_equal(bits_of(ysf[i]), want, err_msg=f"fused: tensor {i} of {n}")


def _fused_list_inputs(dtype):
    """A list with ragged widths, a one-block tensor, an empty tensor, an
    all-zero tensor, one with NaN and infinities, and one spanning several
    units per wave."""
    shapes = [(64, 1024), (48, 272), (1, 16), (0, 32), (200, 4112), (32, 64), (96, 160), (16, 2048)]
    xs = []
    for i, (M, K) in enumerate(shapes):
        t = synthdata.activation_family("outlier", max(M, 1), K, 300 + i, dtype).to(torch.float32)[:M]
        if i == 5:
            t.zero_()
        if i == 6:
            t[3, 7] = float("nan")
            t[50, :16] = float("nan")
            t[10, 9] = float("inf")
            t[11, 0] = -float("inf")
        xs.append(t.to(synthdata.TORCH_DTYPES[dtype]).contiguous())
    return xs


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_qdq_list_fused(orc, dtype):
    """Every tensor's amax and the QDQ of the list in one launch equal the
    oracle's amax of each tensor followed by its QDQ, bit for bit, for every
    mode and both orders; one workspace across the calls."""
    xs = _fused_list_inputs(dtype)
    bits = [raw_bits(x) for x in xs]
    want_a = [orc.amax(b, dtype, "tensor") if b.size else np.zeros(1, np.float32) for b in bits]
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    xd = [dev(x) for x in xs]
    modes = [(r, m, p, o) for (r, m, p) in MODES for o in (("tree", "seq") if r == "4over6" else ("tree",))]
    for (recipe, metric, prec, order), bound in itertools.product(modes, (448, 256)):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, err_order=order)
        ys = [torch.full_like(x, float("nan")) for x in xd]
        ys, amax = fos.fos_qdq_list_fused(xd, outs=ys, workspace=ws, status=status, **kw)
        torch.cuda.synchronize()
        got_a = amax.cpu().numpy().view(np.uint32)
        for i, (b, a) in enumerate(zip(bits, want_a)):
            assert got_a[i] == a.view(np.uint32)[0], f"amax of tensor {i} {kw}"
            if b.size:
                np.testing.assert_array_equal(u_bits(bits_of(ys[i])), u_bits(orc.qdq(b, dtype, a, **kw)),
                                              err_msg=f"tensor {i} {kw}")
    assert int(status.item()) == 0


def test_qdq_list_fused_many_tensors_and_shared_workspace(orc):
    """53 tensors (two launches), with a grouped fused call on the same
    workspace between list calls (the two share the banked slots)."""
    xs = [synthdata.weight(16 + 16 * (i % 3), 64 + 16 * (i % 5), 400 + i, "bf16") for i in range(53)]
    bits = [raw_bits(x) for x in xs]
    want_a = [orc.amax(b, "bf16", "tensor") for b in bits]
    x, offs, _ = synthdata.grouped_tokens(512, 32, 128, 8, seeds=(71, 72, 73, 74), dtype="bf16")
    gb = raw_bits(x)
    starts = np.concatenate([[0], offs[:-1]])
    gam = np.array([orc.amax(gb[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    xd = [dev(t) for t in xs]
    for rep in range(3):
        kw = dict(recipe="4over6", err_metric=("mse", "mae", "mse")[rep], err_prec=("fp16", "exact", "exact")[rep])
        ys, amax = fos.fos_qdq_list_fused(xd, workspace=ws, status=status, **kw)
        _, _, ga, _ = fos.fos_quantize_grouped_fused(dev(x), dev(torch.from_numpy(offs)), workspace=ws,
                                                     status=status, recipe="4over6")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ga.cpu().numpy().view(np.uint32), gam.view(np.uint32))
        got_a = amax.cpu().numpy().view(np.uint32)
        for i in range(53):
            assert got_a[i] == want_a[i].view(np.uint32)[0], f"amax {i}"
            np.testing.assert_array_equal(bits_of(ys[i]), orc.qdq(bits[i], "bf16", want_a[i], **kw), err_msg=f"{i}")
    assert int(status.item()) == 0


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("gran", ["tensor", "row"])
def test_dequantize(orc, out_dtype, gran):
    x = synthdata.activation_family("outlier", 40, 320, 14, "bf16")
    b = raw_bits(x)
    a = orc.amax(b, "bf16", gran)
    q = orc.quantize(b, "bf16", a, recipe="4over6", scale_gran=gran)
    want = orc.dequantize(q["codes"], q["scales"], q["sdec"], gran, out_dtype)
    y = fos.nvfp4_dequantize(dev(torch.from_numpy(q["codes"])), dev(torch.from_numpy(q["scales"])),
                             dev(torch.from_numpy(q["sdec"])), gran, synthdata.TORCH_DTYPES[out_dtype])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u_bits(bits_of(y)), u_bits(want))


# ------------------------------------------------------------------ grouped

@pytest.mark.parametrize("bound", [448, 256])
def test_grouped_small(orc, bound):
    M, pad, K, G = 1024, 64, 272, 16
    x, offs, fac = synthdata.grouped_tokens(M, pad, K, G, seeds=(61, 62, 63, 64))
    b = raw_bits(x)
    starts = np.concatenate([[0], offs[:-1]])
    gam = np.array([orc.amax(b[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    want = orc.quantize_grouped(b, "bf16", offs, gam, recipe="4over6", bound=bound)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales, gsdec = fos.fos_quantize_grouped(dev(x), dev(torch.from_numpy(offs)), dev(torch.from_numpy(gam)),
                                                    recipe="4over6", bound=bound, status=status)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
    np.testing.assert_array_equal(gsdec.cpu().numpy().view(np.uint32), want["group_sdec"].view(np.uint32))
    assert int(status.item()) == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("K", [128, 384])
def test_grouped_flat_units(orc, dtype, K):
    """K a multiple of the unit size: every 16-row band is a whole number of
    units, so the grouped walk runs flat units that cross rows (K = 384: a
    unit spans 5.3 rows of bf16 blocks) but never groups. Both grouped entry
    points equal the oracle's grouped quantize, empty groups and the padding
    tail included."""
    M, pad, G = 512, 48, 12
    x, offs, _ = synthdata.grouped_tokens(M, pad, K, G, seeds=(71, 72, 73, 74), dtype=dtype)
    b = raw_bits(x)
    gam = _group_amaxes(orc, b, dtype, offs)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for metric, prec in (("mse", "exact"), ("mae", "fp16")):
        kw = dict(recipe="4over6", err_metric=metric, err_prec=prec)
        want = orc.quantize_grouped(b, dtype, offs, gam, **kw)
        codes, scales, _ = fos.fos_quantize_grouped(dev(x), dev(torch.from_numpy(offs)), dev(torch.from_numpy(gam)),
                                                    status=status, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{kw}")
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{kw}")
        codes, scales, am, _ = fos.fos_quantize_grouped_fused(dev(x), dev(torch.from_numpy(offs)), workspace=ws,
                                                              status=status, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(am.cpu().numpy().view(np.uint32), gam.view(np.uint32), err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{kw}")
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{kw}")
    assert int(status.item()) == 0


@pytest.mark.parametrize("G", [64, 65, 130])
@pytest.mark.parametrize("K", [128, 272])
def test_grouped_many_groups(orc, G, K):
    """Up to 64 groups are looked up from offsets held one per lane; more go
    through the binary search over offs. Both sides of that limit, with flat
    (K = 128) and per-row (K = 272) units, many empty groups, the plain and
    the fused grouped quantize."""
    M, pad = 1536, 32
    x, offs, _ = synthdata.grouped_tokens(M, pad, K, G, seeds=(91, 92, 93, 94), dtype="bf16")
    b = raw_bits(x)
    gam = _group_amaxes(orc, b, "bf16", offs)
    kw = dict(recipe="4over6", err_metric="mse", err_prec="exact")
    want = orc.quantize_grouped(b, "bf16", offs, gam, **kw)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    codes, scales, _ = fos.fos_quantize_grouped(dev(x), dev(torch.from_numpy(offs)), dev(torch.from_numpy(gam)),
                                                status=status, **kw)
    fc, fs, am, _ = fos.fos_quantize_grouped_fused(dev(x), dev(torch.from_numpy(offs)), workspace=ws, status=status,
                                                   **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
    np.testing.assert_array_equal(am.cpu().numpy().view(np.uint32), gam.view(np.uint32))
    np.testing.assert_array_equal(fc.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(fs.cpu().numpy(), want["scales"])
    assert int(status.item()) == 0


def test_grouped_empty_groups_and_bad_offsets(orc):
    K = 64
    x = synthdata.normal(96, K, 3, "bf16")
    offs = np.array([0, 32, 32, 64, 64], np.int32)
    gam = np.array([5.0, 2.0, 7.0, 3.0, 9.0], np.float32)
    want = orc.quantize_grouped(raw_bits(x), "bf16", offs, gam, recipe="4over6")
    codes, scales, _ = fos.fos_quantize_grouped(dev(x), dev(torch.from_numpy(offs)), dev(torch.from_numpy(gam)),
                                                recipe="4over6")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
    for bad in ([0, 40, 32, 64, 64], [0, 33, 48, 64, 64], [0, 32, 48, 64, 112]):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        fos.fos_quantize_grouped(dev(x), dev(torch.tensor(bad, dtype=torch.int32)), dev(torch.from_numpy(gam)),
                                 recipe="4over6", status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & fos.STATUS_BAD_OFFS


def _group_amaxes(orc, b, dtype, offs):
    starts = np.concatenate([[0], offs[:-1]])
    return np.array([orc.amax(b[s:e], dtype, "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                    np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_grouped_fused(orc, dtype):
    """Group amaxes and the grouped quantize in one launch equal the
    oracle's per-group amaxes followed by its grouped quantize, for every
    mode and both orders. Two inputs with different group scales alternate
    on one workspace, with a per-tensor fused call in between, so a group
    maximum left over from an earlier call would show; the padding rows hold
    large values and NaN that must not count."""
    M, pad, K, G = 1024, 64, 272, 16
    xs, bs, offs_list, gams = [], [], [], []
    for seeds in ((61, 62, 63, 64), (65, 66, 67, 68)):
        x, offs, _ = synthdata.grouped_tokens(M, pad, K, G, seeds=seeds, dtype=dtype)
        xs.append(x)
        bs.append(raw_bits(x))
        offs_list.append(offs)
        gams.append(_group_amaxes(orc, bs[-1], dtype, offs))
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    xd = [dev(x) for x in xs]
    od = [dev(torch.from_numpy(o)) for o in offs_list]
    modes = [(r, m, p, o) for (r, m, p) in MODES for o in (("tree", "seq") if r == "4over6" else ("tree",))]
    for k, ((recipe, metric, prec, order), bound) in enumerate(itertools.product(modes, (448, 256))):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, err_order=order)
        i = k % 2
        codes, scales, gam, gsdec = fos.fos_quantize_grouped_fused(xd[i], od[i], workspace=ws, status=status, **kw)
        torch.cuda.synchronize()
        want = orc.quantize_grouped(bs[i], dtype, offs_list[i], gams[i], **kw)
        np.testing.assert_array_equal(gam.cpu().numpy().view(np.uint32), gams[i].view(np.uint32), err_msg=f"{kw}")
        np.testing.assert_array_equal(gsdec.cpu().numpy().view(np.uint32), want["group_sdec"].view(np.uint32))
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{kw}")
        if k % 3 == 0:  # a per-tensor fused call on the same workspace
            fos.fos_quantize_fused(xd[1 - i][:M], workspace=ws, status=status, **kw)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_grouped_fused_edge_groups(orc):
    """Empty groups, one group, a group holding NaN, an all-zero group, an
    infinite element (S_enc 1 for its group), a ragged K, and offsets that
    break the contract (status bit set)."""
    K = 80
    base = synthdata.normal(160, K, 5, "bf16").to(torch.float32)
    base[100:128] = 0.0            # group 4 of the first case: all zero
    base[40, 3] = float("nan")     # group 1: a NaN
    base[70, 9] = float("inf")     # group 2: inf
    base[150:] = float("nan")      # padding past offs[-1]
    x = base.to(torch.bfloat16)
    b = raw_bits(x)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for offs in ([0, 48, 48, 96, 128, 144], [144], [16, 16, 16, 144], [0, 0, 0]):
        offs = np.array(offs, np.int32)
        gam = _group_amaxes(orc, b, "bf16", offs)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        codes, scales, amax, _ = fos.fos_quantize_grouped_fused(dev(x), dev(torch.from_numpy(offs)), workspace=ws,
                                                                status=status, recipe="4over6")
        torch.cuda.synchronize()
        want = orc.quantize_grouped(b, "bf16", offs, gam, recipe="4over6")
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), gam.view(np.uint32), err_msg=f"{offs}")
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{offs}")
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{offs}")
        assert int(status.item()) == 0
    for bad in ([0, 40, 32, 64, 64], [0, 33, 48, 64, 64], [0, 32, 48, 64, 176]):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        fos.fos_quantize_grouped_fused(dev(x), dev(torch.tensor(bad, dtype=torch.int32)), workspace=ws,
                                       status=status, recipe="4over6")
        torch.cuda.synchronize()
        assert int(status.item()) & fos.STATUS_BAD_OFFS
    # a clean call after the bad ones still matches
    offs = np.array([0, 48, 48, 96, 128, 144], np.int32)
    gam = _group_amaxes(orc, b, "bf16", offs)
    codes, scales, amax, _ = fos.fos_quantize_grouped_fused(dev(x), dev(torch.from_numpy(offs)), workspace=ws,
                                                            recipe="4over6")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), gam.view(np.uint32))
    want = orc.quantize_grouped(b, "bf16", offs, gam, recipe="4over6")
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    with pytest.raises(fos.FosError):
        fos.fos_quantize_grouped_fused(dev(x), dev(torch.zeros(fos.FUSED_MAX_GROUPS + 1, dtype=torch.int32)),
                                       workspace=ws)


# ------------------------------------------------------------------ amax

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_amax(orc, dtype):
    t = synthdata.activation_family("outlier", 96, 1040, 8, dtype).to(torch.float32)
    t[3, 5] = float("nan")
    t[17, :] = float("nan")
    t[40, 7] = -float("inf") if dtype != "fp16" else -60000.0
    t = t.to(synthdata.TORCH_DTYPES[dtype])
    b = raw_bits(t)
    for gran in ("tensor", "row", "band16"):
        got = fos.fos_amax(dev(t), gran)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), orc.amax(b, dtype, gran).view(np.uint32))


# ------------------------------------------------------------------ boundary

def test_empty_inputs(orc):
    for M, K in ((0, 64), (8, 0), (0, 0)):
        x = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        a = torch.ones(1, dtype=torch.float32, device="cuda")
        codes, scales, sdec = fos.fos_quantize(x, a, recipe="4over6")
        y = fos.fos_qdq(x, a, recipe="4over6")
        am = fos.fos_amax(x, "tensor")
        torch.cuda.synchronize()
        assert codes.numel() == 0 and y.numel() == 0
        assert float(am.item()) == 0.0
        assert float(sdec.item()) == orc.global_decode_scale(1.0, 448)


def test_rejects_bad_arguments():
    x = torch.zeros(16, 64, dtype=torch.bfloat16, device="cuda")
    a = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(fos.FosError):
        fos.fos_quantize(torch.zeros(16, 40, dtype=torch.bfloat16, device="cuda"), a)   # K % 16
    with pytest.raises(fos.FosError):
        fos.fos_quantize(torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda"), a, block="16x16")  # M % 16
    with pytest.raises(fos.FosError):
        fos.fos_quantize(x, a, bound=300)
    with pytest.raises(fos.FosError):
        fos.fos_quantize(x, a, block="16x16", err_order="seq")  # the sequential order is 1x16 only
    with pytest.raises(fos.FosError):
        fos.fos_qdq(x, a, block="16x16", err_order="seq")
    flat = torch.zeros(16 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fos.FosError):
        fos.fos_quantize(flat[1:1 + 16 * 64].view(16, 64), a)  # misaligned


def test_runs_on_a_side_stream(orc):
    x = synthdata.normal(128, 512, 9, "bf16")
    amax = orc.amax(raw_bits(x), "bf16", "tensor")
    want = orc.quantize(raw_bits(x), "bf16", amax, recipe="4over6")
    s = torch.cuda.Stream()
    xd, ad = dev(x), dev(torch.from_numpy(amax))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        codes, scales, _ = fos.fos_quantize(xd, ad, recipe="4over6")
    s.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])


def test_fused_calls_on_a_side_stream(orc):
    """The fused entry points launch on the caller's current stream."""
    x = synthdata.activation_family("outlier", 96, 1040, 10, "bf16")
    b = raw_bits(x)
    at, ar = orc.amax(b, "bf16", "tensor"), orc.amax(b, "bf16", "row")
    s = torch.cuda.Stream()
    xd = dev(x)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c1, s1, _, _ = fos.fos_quantize_fused(xd, workspace=ws, recipe="4over6")
        c2, s2, _, _ = fos.fos_quantize_fused(xd, workspace=ws, recipe="4over6", scale_gran="row")
        y, _ = fos.fos_qdq_fused(xd, workspace=ws, recipe="4over6", err_prec="fp16")
    s.synchronize()
    w1 = orc.quantize(b, "bf16", at, recipe="4over6")
    w2 = orc.quantize(b, "bf16", ar, recipe="4over6", scale_gran="row")
    np.testing.assert_array_equal(c1.cpu().numpy(), w1["codes"])
    np.testing.assert_array_equal(s1.cpu().numpy(), w1["scales"])
    np.testing.assert_array_equal(c2.cpu().numpy(), w2["codes"])
    np.testing.assert_array_equal(s2.cpu().numpy(), w2["scales"])
    np.testing.assert_array_equal(bits_of(y), orc.qdq(b, "bf16", at, recipe="4over6", err_prec="fp16"))


def test_fused_calls_replay_in_a_graph(orc):
    """The fused calls allocate nothing and clear nothing with a memset, so a
    captured graph of them replays correctly: three replays over changing
    inputs, with eager work and synchronisation between them, each checked
    against the oracle."""
    M, K = 64, 1040
    xd = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    codes = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    sdec = torch.empty(1, dtype=torch.float32, device="cuda")
    y = torch.empty_like(xd)
    qa = torch.empty(1, dtype=torch.float32, device="cuda")
    xd.copy_(synthdata.normal(M, K, 30, "bf16").to("cuda"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the calls up on the capture stream first
        fos.fos_quantize_fused(xd, codes=codes, scales=scales, amax=amax, sdec=sdec, workspace=ws, recipe="4over6")
        fos.fos_qdq_fused(xd, out=y, amax=qa, workspace=ws, recipe="4over6", err_prec="fp16")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fos.fos_quantize_fused(xd, codes=codes, scales=scales, amax=amax, sdec=sdec, workspace=ws, recipe="4over6")
        fos.fos_qdq_fused(xd, out=y, amax=qa, workspace=ws, recipe="4over6", err_prec="fp16")
    for seed in (31, 32, 33):
        x = synthdata.activation_family("outlier", M, K, seed, "bf16")
        xd.copy_(x.to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        b = raw_bits(x)
        a = orc.amax(b, "bf16", "tensor")
        want = orc.quantize(b, "bf16", a, recipe="4over6")
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32), err_msg=f"{seed}")
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{seed}")
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{seed}")
        np.testing.assert_array_equal(bits_of(y), orc.qdq(b, "bf16", a, recipe="4over6", err_prec="fp16"),
                                      err_msg=f"{seed}")
    assert not ws[256:].any()


# ------------------------------------------------------------------ fused amax + quantize

FUSED_CASES = [((67, 1552), "outlier"), ((256, 1024), "normal"), ((1, 16), "special"), ((96, 1040), "special"),
               ((3, 4096), "uniform"), ((0, 64), "normal")]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_fused_amax_quantize(orc, dtype):
    """One launch for the per-tensor amax and the quantize equals the oracle's
    amax followed by its quantize, for every mode; the workspace comes back
    counters zero after each call, so calls of different sizes can follow
    each other."""
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for (M, K), family in FUSED_CASES:
        x = _family(family, dtype, M, K, 61) if M else torch.empty(0, K, dtype=synthdata.TORCH_DTYPES[dtype])
        b = raw_bits(x)
        want_amax = orc.amax(b, dtype, "tensor")
        for (recipe, metric, prec), bound in itertools.product(MODES, (448, 256)):
            kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound)
            codes, scales, amax, sdec = fos.fos_quantize_fused(dev(x), workspace=ws, status=status, **kw)
            torch.cuda.synchronize()
            want = orc.quantize(b, dtype, want_amax, **kw)
            np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), want_amax.view(np.uint32))
            np.testing.assert_array_equal(sdec.cpu().numpy().view(np.uint32), want["sdec"].view(np.uint32))
            np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{M}x{K} {kw}")
            np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{M}x{K} {kw}")
            assert not ws[256:].any(), "the workspace's counters must be zero after a call"
    assert int(status.item()) == 0


def test_fused_stage_lanes_past_the_end(orc):
    """Small tensors take the one-read fused form, whose waves stage units in
    LDS; a stage lane past the tensor's end holds what an earlier launch
    left there and must not count in the amax. A launch over large values
    fills the stages first, then ragged tensors of small values follow."""
    big = (synthdata.normal(512, 4096, 81, "bf16").to(torch.float32) * 1e30).to(torch.bfloat16)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for dtype, (M, K) in (("bf16", (67, 1552)), ("fp32", (5, 208)), ("fp16", (33, 4112))):
        fos.fos_quantize_fused(dev(big), workspace=ws, status=status, recipe="4over6")
        x = synthdata.normal(M, K, 82, dtype)
        b = raw_bits(x)
        a = orc.amax(b, dtype, "tensor")
        codes, scales, amax, _ = fos.fos_quantize_fused(dev(x), workspace=ws, status=status, recipe="4over6")
        torch.cuda.synchronize()
        want = orc.quantize(b, dtype, a, recipe="4over6")
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32), err_msg=dtype)
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=dtype)
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=dtype)
    assert int(status.item()) == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_qdq_fused(orc, dtype):
    """The per-tensor amax and the fused QDQ in one launch equal the oracle's
    amax followed by its QDQ, for every mode and bound, ragged and empty
    shapes included; the workspace's counters come back zero."""
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for (M, K), family in FUSED_CASES + [((48, 272), "weight")]:
        x = _family(family, dtype, M, K, 63) if M else torch.empty(0, K, dtype=synthdata.TORCH_DTYPES[dtype])
        b = raw_bits(x)
        want_amax = orc.amax(b, dtype, "tensor")
        for (recipe, metric, prec), bound in itertools.product(MODES, (448, 256)):
            kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound)
            y, amax = fos.fos_qdq_fused(dev(x), workspace=ws, status=status, **kw)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), want_amax.view(np.uint32))
            np.testing.assert_array_equal(u_bits(bits_of(y)), u_bits(orc.qdq(b, dtype, want_amax, **kw)),
                                          err_msg=f"{M}x{K} {kw}")
            assert not ws[256:].any(), "the workspace's counters must be zero after a call"
    assert int(status.item()) == 0


def test_fused_phase_timestamps(orc):
    """Diagnostics of the one-read fused quantize: with a timestamp buffer
    set, every wave writes its start, loads-landed, barrier-release and end
    times in that order, rows past the grid stay untouched, and the outputs
    still match the oracle."""
    M, K = 2048, 4096
    x = synthdata.normal(M, K, 91, "bf16")
    b = raw_bits(x)
    buf = torch.zeros(16384, 4, dtype=torch.int64, device="cuda")
    khz = fos.set_phase_timestamps(buf)
    try:
        codes, scales, amax, _ = fos.fos_quantize_fused(dev(x), check=True, recipe="4over6")
        torch.cuda.synchronize()
    finally:
        fos.set_phase_timestamps(None)
    assert khz > 0
    t = buf.cpu().numpy()
    used = t[:, 0] != 0
    n = int(used.sum())
    assert n > 0 and used[:n].all() and not used[n:].any(), "waves 0 .. n-1 write, no other row"
    assert (np.diff(t[:n], axis=1) >= 0).all(), "phases out of order"
    a = orc.amax(b, "bf16", "tensor")
    want = orc.quantize(b, "bf16", a, recipe="4over6")
    np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
    # off again: a later launch writes nothing
    buf.zero_()
    fos.fos_quantize_fused(dev(x), check=True, recipe="4over6")
    torch.cuda.synchronize()
    assert not buf.any()


def test_qdq_fused_stage_lanes_past_the_end(orc):
    """As for the fused quantize: stage lanes past a ragged tensor's end hold
    an earlier launch's values, which must not count in the amax."""
    big = (synthdata.normal(512, 4096, 83, "bf16").to(torch.float32) * 1e30).to(torch.bfloat16)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for dtype, (M, K) in (("bf16", (67, 1552)), ("fp32", (5, 208)), ("fp16", (33, 4112))):
        fos.fos_qdq_fused(dev(big), workspace=ws, recipe="4over6")
        x = synthdata.normal(M, K, 84, dtype)
        b = raw_bits(x)
        a = orc.amax(b, dtype, "tensor")
        y, amax = fos.fos_qdq_fused(dev(x), workspace=ws, recipe="4over6", err_prec="fp16")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32), err_msg=dtype)
        np.testing.assert_array_equal(u_bits(bits_of(y)), u_bits(orc.qdq(b, dtype, a, recipe="4over6", err_prec="fp16")),
                                      err_msg=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_fused_row_amax_quantize(orc, dtype):
    """Per-row amaxes and the quantize in one launch equal the oracle's
    per-row amax followed by its per-row quantize, for every mode and bound:
    rows of zeros, a row of NaN, an infinite element, ragged and long rows."""
    cases = [((67, 1552), "outlier"), ((96, 1040), "special"), ((1, 16), "normal"), ((5, 14336), "normal"),
             ((0, 64), "normal")]
    for (M, K), family in cases:
        x = _family(family, dtype, M, K, 65) if M else torch.empty(0, K, dtype=synthdata.TORCH_DTYPES[dtype])
        if M >= 67:
            t = x.to(torch.float32)
            t[10, :] = float("nan")
            t[20, 3] = float("inf") if dtype != "fp16" else 60000.0
            x = t.to(synthdata.TORCH_DTYPES[dtype])
        b = raw_bits(x)
        want_amax = orc.amax(b, dtype, "row")
        for (recipe, metric, prec), bound in itertools.product(MODES, (448, 256)):
            kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, scale_gran="row")
            codes, scales, amax, sdec = fos.fos_quantize_fused(dev(x), **kw)
            torch.cuda.synchronize()
            want = orc.quantize(b, dtype, want_amax, **kw)
            np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), want_amax.view(np.uint32))
            np.testing.assert_array_equal(sdec.cpu().numpy().view(np.uint32), want["sdec"].view(np.uint32))
            np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{M}x{K} {kw}")
            np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{M}x{K} {kw}")


def test_fused_nan_inf_tensors(orc):
    """NaN-dropping amax inside the fused launch: scattered NaN, an all-NaN
    tensor (amax 0, S_enc 1) and an infinite element (S_enc 1)."""
    base = synthdata.normal(64, 256, 62, "bf16").to(torch.float32)
    cases = []
    t = base.clone(); t[5, 7] = float("nan"); t[60, :] = float("nan"); cases.append(t)
    cases.append(torch.full((32, 64), float("nan")))
    t = base.clone(); t[10, 3] = float("inf"); cases.append(t)
    for t in cases:
        x = t.to(torch.bfloat16)
        b = raw_bits(x)
        a = orc.amax(b, "bf16", "tensor")
        codes, scales, amax, sdec = fos.fos_quantize_fused(dev(x), recipe="4over6")
        torch.cuda.synchronize()
        want = orc.quantize(b, "bf16", a, recipe="4over6")
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])


# ------------------------------------------------------------------ sequential order, wider QDQ

SEQ_MODES = [("4over6", m, p) for m in ("mae", "mse") for p in ("exact", "fp16")]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_sequential_order_every_entry(orc, dtype):
    """The sequential error order through quantize (per tensor and per row),
    QDQ, the grouped call and the fused call, on ragged shapes."""
    M, K = 67, 1552
    x = _family("outlier", dtype, M, K, 71)
    b = raw_bits(x)
    am = {"tensor": orc.amax(b, dtype, "tensor"), "row": orc.amax(b, dtype, "row")}
    for (recipe, metric, prec), bound in itertools.product(SEQ_MODES, (448, 256)):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, err_order="seq")
        for gran in ("tensor", "row"):
            assert_quant_equal(orc, x, dtype, am[gran], label="seq", scale_gran=gran, **kw)
            y = fos.fos_qdq(dev(x), dev(torch.from_numpy(am[gran])), scale_gran=gran, **kw)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(u_bits(bits_of(y)), u_bits(orc.qdq(b, dtype, am[gran], scale_gran=gran, **kw)))
        codes, scales, amax, _ = fos.fos_quantize_fused(dev(x), **kw)
        torch.cuda.synchronize()
        want = orc.quantize(b, dtype, am["tensor"], **kw)
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
    # grouped
    offs = np.array([16, 16, 48, 64], np.int32)
    gam = np.array([orc.amax(b[s:e], dtype, "tensor")[0] if e > s else 0.0
                    for s, e in zip([0, 16, 16, 48], offs)], np.float32)
    for recipe, metric, prec in SEQ_MODES:
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, err_order="seq")
        want = orc.quantize_grouped(b, dtype, offs, gam, **kw)
        codes, scales, _ = fos.fos_quantize_grouped(dev(x), dev(torch.from_numpy(offs)), dev(torch.from_numpy(gam)),
                                                    **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("block,gran", [("1x16", "tensor"), ("1x16", "row"), ("16x16", "tensor"), ("16x16", "row")])
def test_qdq_every_dtype_block_and_granularity(orc, dtype, block, gran):
    """Fused QDQ beyond the page's bf16/fp16 1x16 per-tensor path: fp32,
    row-scaled and 16x16, against the oracle's QDQ, as one tensor and as a
    list of tensors of different shapes."""
    shapes = [(48, 272), (16, 16), (96, 1040)]
    xs = [_family(f, dtype, M, K, 80 + i) for i, ((M, K), f) in enumerate(zip(shapes, ("weight", "outlier", "special")))]
    bs = [raw_bits(x) for x in xs]
    mode = "tensor" if gran == "tensor" else ("band16" if block == "16x16" else "row")
    ams = [orc.amax(b, dtype, mode) for b in bs]
    for (recipe, metric, prec), bound in itertools.product(MODES, (448, 256)):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, block=block, scale_gran=gran)
        ys = fos.fos_qdq_list([dev(x) for x in xs], [dev(torch.from_numpy(a)) for a in ams], **kw)
        y0 = fos.fos_qdq(dev(xs[0]), dev(torch.from_numpy(ams[0])), **kw)
        torch.cuda.synchronize()
        for i in range(len(xs)):
            np.testing.assert_array_equal(u_bits(bits_of(ys[i])), u_bits(orc.qdq(bs[i], dtype, ams[i], **kw)),
                                          err_msg=f"{i} {kw}")
        np.testing.assert_array_equal(u_bits(bits_of(y0)), u_bits(orc.qdq(bs[0], dtype, ams[0], **kw)))


# ------------------------------------------------------------------ columnwise

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("shape,family", [((48, 272), "outlier"), ((16, 16), "special"), ((96, 1040), "normal"),
                                          ((32, 4096), "special"), ((272, 48), "weight"), ((512, 208), "normal"),
                                          ((528, 80), "outlier")])
def test_columnwise_is_quantize_of_the_transpose(orc, dtype, shape, family):
    """fos_quantize_columnwise(x) equals the oracle's quantize of x^T, every
    mode, both bounds and both error orders: ragged column strips, a partial
    last 256-row group (528 rows), whole aligned groups (512 rows, the
    16-byte store path) and rows that leave the xT runs 8-byte aligned."""
    M, K = shape
    x = _family(family, dtype, M, K, 73)
    if family == "special":
        x = x.to(torch.float32)
        x[3, 5] = float("nan")
        x[7, 9] = float("-inf")
        x = x.to(synthdata.TORCH_DTYPES[dtype])
    b = raw_bits(x)
    bt = np.ascontiguousarray(b.T)
    a = orc.amax(b, dtype, "tensor")
    modes = [(r, m, p, o) for (r, m, p) in MODES for o in (("tree", "seq") if r == "4over6" else ("tree",))]
    for (recipe, metric, prec, order), bound in itertools.product(modes, (448, 256)):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, err_order=order)
        codes, scales, sdec = fos.fos_quantize_columnwise(dev(x), dev(torch.from_numpy(a)), **kw)
        torch.cuda.synchronize()
        want = orc.quantize(bt, dtype, a, **kw)
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{shape} {kw}")
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{shape} {kw}")
        np.testing.assert_array_equal(sdec.cpu().numpy().view(np.uint32), want["sdec"].view(np.uint32))
