"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole tensor goes through the library in one call, and
the oracle recomputes sampled rows (1x16; per-row independence given the
global scale) or sampled 16-row bands (16x16). Global amaxes are compared in
full. Every knob combination of each workload is run; reused output buffers
are filled with a sentinel byte before each call. One mode per workload is
compared on the whole tensor in test_gpu_fullsize_whole.py.

Workloads: the dense activation tensor (bf16 8192x4096, four data families),
the 16x16 weights (bf16 4096x14336, fp32 4096x4096), the fused-QDQ expert
list (8 x 2048x7168, bf16 and fp16) and the grouped MoE tokens
(65536 + 4096 padding rows x 7168, 64 groups).
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
BOUNDS = (448, 256)


def sample_rows(M, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, M - 1], rng.integers(0, M, n), np.asarray(extra, np.int64)])
    return np.unique(rows.astype(np.int64))


def check_amax(orc, x_dev, bits, dtype, gran):
    got = fos.fos_amax(x_dev, gran)
    torch.cuda.synchronize()
    want = orc.amax(bits, dtype, gran)
    np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32), err_msg=f"amax {gran}")
    return want


# ------------------------------------------------------------------ dense activations

@pytest.mark.parametrize("family", synthdata.ACTIVATION_FAMILIES)
def test_dense_activation_8192x4096(orc, family):
    M, K = 8192, 4096
    seed = 21 + synthdata.ACTIVATION_FAMILIES.index(family)
    x = synthdata.activation_family(family, M, K, seed, "bf16")
    bits = raw_bits(x)
    xd = x.to("cuda")
    am = {"tensor": check_amax(orc, xd, bits, "bf16", "tensor"), "row": check_amax(orc, xd, bits, "bf16", "row")}
    rows = sample_rows(M, 48, seed, extra=range(8))
    codes = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
    for (recipe, metric, prec), bound, gran in itertools.product(MODES, BOUNDS, ("tensor", "row")):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, scale_gran=gran)
        a = am[gran]
        codes.fill_(0xA5)  # sentinel: a block left unwritten shows
        scales.fill_(0xA5)
        _, _, sdec = fos.fos_quantize(xd, torch.from_numpy(a).to("cuda"), codes=codes, scales=scales, **kw)
        torch.cuda.synchronize()
        want = orc.quantize(bits[rows], "bf16", a if gran == "tensor" else a[rows], **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"], err_msg=f"scales {family} {kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"], err_msg=f"codes {family} {kw}")
        sd = sdec.cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(sd if gran == "tensor" else sd[rows], want["sdec"].view(np.uint32))


# ------------------------------------------------------------------ 16x16 weights

@pytest.mark.parametrize("dtype,M,K,seed", [("bf16", 4096, 14336, 31), ("fp32", 4096, 4096, 32)])
def test_weights_16x16(orc, dtype, M, K, seed):
    x = synthdata.weight(M, K, seed, dtype)
    bits = raw_bits(x)
    xd = x.to("cuda")
    am = {"tensor": check_amax(orc, xd, bits, dtype, "tensor"), "row": check_amax(orc, xd, bits, dtype, "band16")}
    bands = np.unique(np.concatenate([[0, M // 16 - 1], np.random.default_rng(seed).integers(0, M // 16, 3)]))
    rows = (bands[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
    codes = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for (recipe, metric, prec), bound, gran in itertools.product(MODES, BOUNDS, ("tensor", "row")):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, scale_gran=gran, block="16x16")
        a = am[gran]
        codes.fill_(0xA5)  # sentinel: a block left unwritten shows
        scales.fill_(0xA5)
        fos.fos_quantize(xd, torch.from_numpy(a).to("cuda"), codes=codes, scales=scales, status=status, **kw)
        torch.cuda.synchronize()
        want = orc.quantize(bits[rows], dtype, a if gran == "tensor" else a[rows], **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"], err_msg=f"scales {dtype} {kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"], err_msg=f"codes {dtype} {kw}")
    assert int(status.item()) == 0  # band amaxes are uniform within each tile


# ------------------------------------------------------------------ fused QDQ over the expert list

@pytest.mark.parametrize("order", ["tree", "seq"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_qdq_expert_list_8x2048x7168(orc, dtype, order):
    lst = synthdata.expert_weight_list(8, 2048, 7168, 40, dtypes=(dtype,))[dtype]
    bits = [raw_bits(t) for t in lst]
    xs = [t.to("cuda") for t in lst]
    ams = [orc.amax(b, dtype, "tensor") for b in bits]
    ams_d = [torch.from_numpy(a).to("cuda") for a in ams]
    ys = [torch.empty_like(t) for t in xs]
    rows = [sample_rows(2048, 12, 100 + i) for i in range(8)]
    modes = MODES if order == "tree" else [m for m in MODES if m[0] == "4over6"]
    for (recipe, metric, prec), bound in itertools.product(modes, BOUNDS):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound, err_order=order)
        fos.fos_qdq_list(xs, ams_d, outs=ys, **kw)
        torch.cuda.synchronize()
        for i in range(8):
            want = orc.qdq(bits[i][rows[i]], dtype, ams[i], **kw)
            got = raw_bits(ys[i].cpu())[rows[i]]
            np.testing.assert_array_equal(got, want, err_msg=f"tensor {i} {kw}")


# ------------------------------------------------------------------ grouped MoE tokens

def test_grouped_moe_65536x7168(orc):
    M, pad, K, G = 65536, 4096, 7168, 64
    x, offs, _ = synthdata.grouped_tokens(M, pad, K, G)
    bits = raw_bits(x)
    starts = np.concatenate([[0], offs[:-1]]).astype(np.int64)
    gam = np.array([orc.amax(bits[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    group_of_row = np.searchsorted(offs, np.arange(M), side="right")
    edges = [r for s, e in zip(starts, offs) if e > s for r in (s, e - 1)]
    rows = sample_rows(M, 96, 55, extra=edges)
    xd = x.to("cuda")
    codes = torch.empty(M + pad, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M + pad, K // 16, dtype=torch.uint8, device="cuda")
    gsdec = torch.empty(G, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for bound in BOUNDS:
        kw = dict(recipe="4over6", err_metric="mse", err_prec="exact", bound=bound)
        codes.fill_(0xA5)  # sentinel: a block left unwritten shows
        scales.fill_(0xA5)
        fos.fos_quantize_grouped(xd, torch.from_numpy(offs).to("cuda"), torch.from_numpy(gam).to("cuda"),
                                 codes=codes, scales=scales, group_sdec=gsdec, status=status, **kw)
        torch.cuda.synchronize()
        # rows of group g quantize like a per-row tensor whose row amax is A_g
        want = orc.quantize(bits[rows], "bf16", gam[group_of_row[rows]], scale_gran="row", **kw)
        c = codes.cpu().numpy()
        s = scales.cpu().numpy()
        np.testing.assert_array_equal(s[rows], want["scales"], err_msg=f"scales bound {bound}")
        np.testing.assert_array_equal(c[rows], want["codes"], err_msg=f"codes bound {bound}")
        assert not c[M:].any() and not s[M:].any(), "padding rows must be zero"
        want_sdec = np.array([orc.global_decode_scale(float(a), bound) for a in gam], np.float32)
        np.testing.assert_array_equal(gsdec.cpu().numpy().view(np.uint32), want_sdec.view(np.uint32))
        assert int(status.item()) == 0


def test_grouped_fused_moe_65536x7168(orc):
    """Group amaxes and the grouped quantize in one launch on the full MoE
    token tensor (64 groups, 4096 padding rows of garbage and NaN): all 64
    group amaxes in full, sampled rows (every group's first and last row
    included) against the oracle, both bounds."""
    M, pad, K, G = 65536, 4096, 7168, 64
    x, offs, _ = synthdata.grouped_tokens(M, pad, K, G)
    bits = raw_bits(x)
    starts = np.concatenate([[0], offs[:-1]]).astype(np.int64)
    gam = np.array([orc.amax(bits[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    group_of_row = np.searchsorted(offs, np.arange(M), side="right")
    edges = [r for s, e in zip(starts, offs) if e > s for r in (s, e - 1)]
    rows = sample_rows(M, 96, 56, extra=edges)
    xd = x.to("cuda")
    od = torch.from_numpy(offs).to("cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for bound in BOUNDS:
        kw = dict(recipe="4over6", err_metric="mse", err_prec="exact", bound=bound)
        codes, scales, amax, gsdec = fos.fos_quantize_grouped_fused(xd, od, status=status, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), gam.view(np.uint32))
        want = orc.quantize(bits[rows], "bf16", gam[group_of_row[rows]], scale_gran="row", **kw)
        c = codes.cpu().numpy()
        s = scales.cpu().numpy()
        np.testing.assert_array_equal(s[rows], want["scales"], err_msg=f"scales bound {bound}")
        np.testing.assert_array_equal(c[rows], want["codes"], err_msg=f"codes bound {bound}")
        assert not c[M:].any() and not s[M:].any(), "padding rows must be zero"
        want_sdec = np.array([orc.global_decode_scale(float(a), bound) for a in gam], np.float32)
        np.testing.assert_array_equal(gsdec.cpu().numpy().view(np.uint32), want_sdec.view(np.uint32))
    assert int(status.item()) == 0


def test_fused_dense_activation_8192x4096(orc):
    """The fused amax + quantize on the full dense activation tensor, every
    mode, with one workspace across calls of two sizes."""
    M, K = 8192, 4096
    x = synthdata.activation_family("outlier", M, K, 23, "bf16")
    bits = raw_bits(x)
    xd = x.to("cuda")
    a = orc.amax(bits, "bf16", "tensor")
    rows = sample_rows(M, 48, 23)
    small = synthdata.normal(48, 1040, 5, "bf16")
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for (recipe, metric, prec), bound in itertools.product(MODES, BOUNDS):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound)
        codes, scales, amax, _ = fos.fos_quantize_fused(xd, workspace=ws, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        want = orc.quantize(bits[rows], "bf16", a, **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"], err_msg=f"{kw}")
        c2, s2, _, _ = fos.fos_quantize_fused(small.to("cuda"), workspace=ws, **kw)
        torch.cuda.synchronize()
        w2 = orc.quantize(raw_bits(small), "bf16", orc.amax(raw_bits(small), "bf16", "tensor"), **kw)
        np.testing.assert_array_equal(c2.cpu().numpy(), w2["codes"])
        np.testing.assert_array_equal(s2.cpu().numpy(), w2["scales"])
    assert not ws[256:].any()


@pytest.mark.parametrize("dtype,M,K", [("fp32", 4096, 4096), ("fp32", 4096, 4112), ("fp16", 8192, 4096),
                                       ("fp16", 8192, 4112)])
def test_fused_at_the_one_read_capacity(orc, dtype, M, K):
    """The fused amax + quantize right at the capacity of its one-read form
    (fp32 4096x4096 and fp16 8192x4096 fill it exactly) and just past it
    (K = 4112: the two-read form); sampled rows against the oracle."""
    x = synthdata.activation_family("outlier", M, K, 27, dtype)
    bits = raw_bits(x)
    xd = x.to("cuda")
    a = orc.amax(bits, dtype, "tensor")
    rows = sample_rows(M, 32, 27)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for recipe, metric, prec in (("4over6", "mse", "exact"), ("4over6", "mae", "fp16")):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec)
        codes, scales, amax, _ = fos.fos_quantize_fused(xd, workspace=ws, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        want = orc.quantize(bits[rows], dtype, a, **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"], err_msg=f"{kw}")
    assert not ws[256:].any()


@pytest.mark.parametrize("dtype,M,K", [("bf16", 8192, 4096), ("bf16", 8192, 4112), ("fp32", 4096, 4096),
                                       ("fp32", 4096, 4112)])
def test_qdq_fused_at_the_one_read_capacity(orc, dtype, M, K):
    """The fused amax + QDQ right at the capacity of its one-read launch and
    just past it (K = 4112: the amax launch, then the QDQ launch); sampled
    rows against the oracle's QDQ with the oracle's amax."""
    x = synthdata.activation_family("outlier", M, K, 29, dtype)
    bits = raw_bits(x)
    xd = x.to("cuda")
    a = orc.amax(bits, dtype, "tensor")
    rows = sample_rows(M, 32, 29)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for recipe, metric, prec in (("4over6", "mse", "fp16"), ("4over6", "mae", "exact"), ("nvfp4", "mse", "exact")):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec)
        y, amax = fos.fos_qdq_fused(xd, workspace=ws, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        got = raw_bits(y.cpu())[rows]
        want = orc.qdq(bits[rows], dtype, a, **kw)
        if dtype == "fp32":  # compare bits (signed zeros included)
            got, want = got.view(np.uint32), want.view(np.uint32)
        np.testing.assert_array_equal(got, want, err_msg=f"{kw}")
    assert not ws[256:].any()


@pytest.mark.parametrize("family", ["outlier", "special"])
def test_fused_row_dense_activation_8192x4096(orc, family):
    """The fused per-row amax + quantize on the full dense activation tensor
    (the special family's first rows are all zero); the amaxes in full,
    sampled rows against the oracle."""
    M, K = 8192, 4096
    x = synthdata.activation_family(family, M, K, 24, "bf16")
    bits = raw_bits(x)
    a = orc.amax(bits, "bf16", "row")
    rows = sample_rows(M, 48, 24, extra=range(8))
    for recipe, metric, prec in (("4over6", "mse", "exact"), ("4over6", "mae", "fp16"), ("nvfp4", "mse", "exact")):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, scale_gran="row")
        codes, scales, amax, _ = fos.fos_quantize_fused(x.to("cuda"), **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        want = orc.quantize(bits[rows], "bf16", a[rows], **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"], err_msg=f"{kw}")


@pytest.mark.parametrize("dtype,M,K", [("bf16", 20000, 512), ("bf16", 300, 4096), ("bf16", 300, 4112),
                                       ("fp32", 300, 2048), ("fp32", 300, 2064), ("fp16", 5000, 1040)])
def test_fused_row_stage_limit_and_many_rows(orc, dtype, M, K):
    """The fused per-row amax + quantize with several rows per wave (the
    staged rows pipeline into each other) and with rows exactly at the 8 KiB
    stage (bf16 K = 4096, fp32 K = 2048) and just past it (the read-then-walk
    form); every amax, and sampled rows, against the oracle."""
    x = synthdata.activation_family("outlier", M, K, 33, dtype)
    bits = raw_bits(x)
    a = orc.amax(bits, dtype, "row")
    rows = sample_rows(M, 40, 33)
    kw = dict(recipe="4over6", err_metric="mse", err_prec="exact", scale_gran="row")
    codes, scales, amax, sdec = fos.fos_quantize_fused(x.to("cuda"), **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
    want = orc.quantize(bits[rows], dtype, a[rows], **kw)
    np.testing.assert_array_equal(sdec.cpu().numpy()[rows].view(np.uint32), want["sdec"].view(np.uint32))
    np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"])
    np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"])


def test_fused_beyond_one_read_16384x4096(orc):
    """A tensor too large for the one-read fused form (twice the dense
    activation tensor) takes the two-read form; sampled rows against the
    oracle, for the standard recipe and four-over-six."""
    M, K = 16384, 4096
    x = synthdata.activation_family("outlier", M, K, 25, "bf16")
    bits = raw_bits(x)
    xd = x.to("cuda")
    a = orc.amax(bits, "bf16", "tensor")
    rows = sample_rows(M, 48, 25)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for recipe, metric, prec in (("nvfp4", "mse", "exact"), ("4over6", "mse", "exact"), ("4over6", "mae", "fp16")):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec)
        codes, scales, amax, _ = fos.fos_quantize_fused(xd, workspace=ws, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        want = orc.quantize(bits[rows], "bf16", a, **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[rows], want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[rows], want["codes"], err_msg=f"{kw}")
    assert not ws[256:].any()


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("gran", ["tensor", "row"])
def test_dequantize_8192x4096(orc, out_dtype, gran):
    """nvfp4_dequantize of the dense-activation shape from random codes (every
    nibble value) and random finite E4M3 scales, in the launch configuration
    the benchmark times; sampled rows against the oracle's decode."""
    M, K = 8192, 4096
    codes = synthdata.random_packed_codes(M, K, 91)
    scales = synthdata.random_block_scales(M, K, 92)
    rng = np.random.default_rng(93)
    if gran == "tensor":
        sdec = np.array([0.37], np.float32)
    else:
        sdec = (10.0 ** rng.uniform(-3, 3, M)).astype(np.float32)
    y = fos.nvfp4_dequantize(torch.from_numpy(codes).to("cuda"), torch.from_numpy(scales).to("cuda"),
                             torch.from_numpy(sdec).to("cuda"), gran, synthdata.TORCH_DTYPES[out_dtype])
    torch.cuda.synchronize()
    rows = sample_rows(M, 64, 94)
    want = orc.dequantize(codes[rows], scales[rows], sdec if gran == "tensor" else sdec[rows], gran, out_dtype)
    got = raw_bits(y.cpu())[rows]
    view = np.uint32 if out_dtype == "fp32" else np.uint16
    np.testing.assert_array_equal(np.ascontiguousarray(got).view(view), np.ascontiguousarray(want).view(view))


def test_columnwise_dense_activation_8192x4096(orc):
    """The transposed operand of the dense activation tensor at full size:
    sampled columns of x (rows of x^T) against the oracle's quantize of the
    transpose, every mode."""
    M, K = 8192, 4096
    x = synthdata.activation_family("outlier", M, K, 23, "bf16")
    bits = raw_bits(x)
    a = orc.amax(bits, "bf16", "tensor")
    cols = sample_rows(K, 48, 77)
    xt_rows = np.ascontiguousarray(bits[:, cols].T)
    xd = x.to("cuda")
    for (recipe, metric, prec), bound in itertools.product(MODES, BOUNDS):
        kw = dict(recipe=recipe, err_metric=metric, err_prec=prec, bound=bound)
        codes, scales, _ = fos.fos_quantize_columnwise(xd, torch.from_numpy(a).to("cuda"), **kw)
        torch.cuda.synchronize()
        want = orc.quantize(xt_rows, "bf16", a, **kw)
        np.testing.assert_array_equal(scales.cpu().numpy()[cols], want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(codes.cpu().numpy()[cols], want["codes"], err_msg=f"{kw}")


def test_columnwise_several_tiles_per_wave_16384x8192(orc):
    """A tensor with more 256x64 tiles than the grid has waves (16384 x 8192
    bf16: 8192 tiles), so each wave walks several tiles: sampled columns
    against the oracle's quantize of the transpose."""
    M, K = 16384, 8192
    x = synthdata.activation_family("normal", M, K, 29, "bf16")
    bits = raw_bits(x)
    a = orc.amax(bits, "bf16", "tensor")
    cols = sample_rows(K, 40, 78, extra=[63, 64])
    xt_rows = np.ascontiguousarray(bits[:, cols].T)
    codes, scales, _ = fos.fos_quantize_columnwise(x.to("cuda"), torch.from_numpy(a).to("cuda"), recipe="4over6")
    torch.cuda.synchronize()
    want = orc.quantize(xt_rows, "bf16", a, recipe="4over6")
    np.testing.assert_array_equal(scales.cpu().numpy()[cols], want["scales"])
    np.testing.assert_array_equal(codes.cpu().numpy()[cols], want["codes"])
