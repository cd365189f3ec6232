"""GPU parity on whole tensors at the workloads' full sizes: every output
element compared with the oracle as integer views at zero tolerance (the
Megatron-LM PR "Fuse NVFP4 fake-QAT quantize-dequantize with CuTe DSL",
"Validation": integer views, no tolerance). The outputs are filled with a
sentinel byte before each call, so a row or block that a kernel never writes
shows as a mismatch.

One representative mode per workload runs here on the whole tensor (the
knob sweeps run on sampled rows in test_gpu_fullsize.py):
  - dense activation bf16 8192x4096, all four data families: per-tensor MSE
    exact 448 and MAE FP16-error 448, and the one-launch fused amax +
    quantize (the benchmark's kernel) in MSE exact 448;
  - 16x16 weights bf16 4096x14336 and fp32 4096x4096: per-tensor MSE exact
    448;
  - the fused-QDQ expert list 8 x 2048x7168, bf16 and fp16: MSE FP16-error
    448, with the amaxes given and with them computed in the same launch;
  - the grouped MoE tokens 65536 (+4096 padding) x 7168, 64 groups: MSE
    exact at bounds 448 and 256, and the fused group amaxes at 448.
"""
import numpy as np
import pytest
import torch

import nvfp4_adaptive_block_amd as fos
import synthdata
from synthdata import raw_bits

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _eq(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.cpu().numpy() if got.dtype == torch.uint8 else raw_bits(got.cpu())
    w = np.ascontiguousarray(want)
    if g.dtype == np.float32:
        g, w = g.view(np.uint32), w.view(np.uint32)
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    if bad.size:
        i = int(bad[0])
        K = g.shape[-1]
        pytest.fail(f"{what}: {bad.size} of {g.size} elements differ; first at row {i // K}, column {i % K}: "
                    f"got 0x{int(g.reshape(-1)[i]):x}, want 0x{int(w.reshape(-1)[i]):x}")


@pytest.mark.parametrize("family", synthdata.ACTIVATION_FAMILIES)
def test_dense_activation_whole(orc, family):
    M, K = 8192, 4096
    seed = 21 + synthdata.ACTIVATION_FAMILIES.index(family)
    x = synthdata.activation_family(family, M, K, seed, "bf16")
    bits = raw_bits(x)
    xd = x.to("cuda")
    a = orc.amax(bits, "bf16", "tensor")
    ad = torch.from_numpy(a).to("cuda")
    codes = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
    for metric, prec in (("mse", "exact"), ("mae", "fp16")):
        kw = dict(recipe="4over6", err_metric=metric, err_prec=prec, bound=448)
        codes.fill_(SENTINEL)
        scales.fill_(SENTINEL)
        fos.fos_quantize(xd, ad, codes=codes, scales=scales, **kw)
        want = orc.quantize(bits, "bf16", a, **kw)
        _eq(scales, want["scales"], f"scales {family} {kw}")
        _eq(codes, want["codes"], f"codes {family} {kw}")
        if metric == "mse":  # the benchmark's one-launch fused amax + quantize
            codes.fill_(SENTINEL)
            scales.fill_(SENTINEL)
            _, _, amax, _ = fos.fos_quantize_fused(xd, codes=codes, scales=scales, check=True, **kw)
            _eq(amax, a, f"fused amax {family}")
            _eq(scales, want["scales"], f"fused scales {family} {kw}")
            _eq(codes, want["codes"], f"fused codes {family} {kw}")


@pytest.mark.parametrize("dtype,M,K,seed", [("bf16", 4096, 14336, 31), ("fp32", 4096, 4096, 32)])
def test_weights_16x16_whole(orc, dtype, M, K, seed):
    x = synthdata.weight(M, K, seed, dtype)
    bits = raw_bits(x)
    a = orc.amax(bits, dtype, "tensor")
    codes = torch.full((M, K // 2), SENTINEL, dtype=torch.uint8, device="cuda")
    scales = torch.full((M, K // 16), SENTINEL, dtype=torch.uint8, device="cuda")
    kw = dict(recipe="4over6", block="16x16", err_metric="mse", err_prec="exact", bound=448)
    fos.fos_quantize(x.to("cuda"), torch.from_numpy(a).to("cuda"), codes=codes, scales=scales, **kw)
    want = orc.quantize(bits, dtype, a, **kw)
    _eq(scales, want["scales"], f"scales {dtype}")
    _eq(codes, want["codes"], f"codes {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_qdq_expert_list_whole(orc, dtype):
    lst = synthdata.expert_weight_list(8, 2048, 7168, 40, dtypes=(dtype,))[dtype]
    bits = [raw_bits(t) for t in lst]
    xs = [t.to("cuda") for t in lst]
    ams = [orc.amax(b, dtype, "tensor") for b in bits]
    ys = [torch.full_like(t, float("nan")) for t in xs]  # sentinel: NaN never appears in a QDQ output
    kw = dict(recipe="4over6", err_metric="mse", err_prec="fp16", bound=448)
    fos.fos_qdq_list(xs, [torch.from_numpy(a).to("cuda") for a in ams], outs=ys, **kw)
    want = [orc.qdq(bits[i], dtype, ams[i], **kw) for i in range(8)]
    for i in range(8):
        _eq(ys[i], want[i], f"tensor {i} {dtype}")
    # every amax and the QDQ in one launch
    ys = [torch.full_like(t, float("nan")) for t in xs]
    _, amax = fos.fos_qdq_list_fused(xs, outs=ys, check=True, **kw)
    _eq(amax, np.concatenate(ams), f"fused list amaxes {dtype}")
    for i in range(8):
        _eq(ys[i], want[i], f"fused list tensor {i} {dtype}")


def test_grouped_moe_whole(orc):
    M, pad, K, G = 65536, 4096, 7168, 64
    x, offs, _ = synthdata.grouped_tokens(M, pad, K, G)
    bits = raw_bits(x)
    starts = np.concatenate([[0], offs[:-1]]).astype(np.int64)
    gam = np.array([orc.amax(bits[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    xd = x.to("cuda")
    od = torch.from_numpy(offs).to("cuda")
    gd = torch.from_numpy(gam).to("cuda")
    codes = torch.empty(M + pad, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M + pad, K // 16, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for bound in (448, 256):
        kw = dict(recipe="4over6", err_metric="mse", err_prec="exact", bound=bound)
        want = orc.quantize_grouped(bits, "bf16", offs, gam, **kw)
        codes.fill_(SENTINEL)
        scales.fill_(SENTINEL)
        fos.fos_quantize_grouped(xd, od, gd, codes=codes, scales=scales, status=status, **kw)
        _eq(scales, want["scales"], f"grouped scales bound {bound}")
        _eq(codes, want["codes"], f"grouped codes bound {bound}")
        if bound == 448:  # the fused group amaxes, one launch
            codes.fill_(SENTINEL)
            scales.fill_(SENTINEL)
            _, _, amax, _ = fos.fos_quantize_grouped_fused(xd, od, codes=codes, scales=scales, check=True, **kw)
            _eq(amax, gam, "fused group amaxes")
            _eq(scales, want["scales"], "fused grouped scales")
            _eq(codes, want["codes"], "fused grouped codes")
    torch.cuda.synchronize()
    assert int(status.item()) == 0
