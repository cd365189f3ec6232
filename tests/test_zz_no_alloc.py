"""The allocation-free grouped fused entry point, called through the C ABI,
against the workspace-taking entry point it varies: two calls in a row on
the library-held workspace, the second with a smaller input (fewer rows,
narrower rows, fewer groups), each bit-exact with
fos_quantize_grouped_fused on a fresh workspace, and with the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_adaptive_block_amd as fos
import synthdata
from synthdata import raw_bits

pytestmark = pytest.mark.gpu


def _group_amaxes(orc, b, dtype, offs):
    starts = np.concatenate([[0], offs[:-1]])
    return np.array([orc.amax(b[s:e], dtype, "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                    np.float32)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_the_workspace_entry_point(orc):
    lib = fos.load_library()
    cfg = fos.config(recipe="4over6", err_metric="mse", err_prec="exact", bound=448)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # a larger call, then a smaller one: fewer rows, narrower rows, fewer groups
    cases = [((4096, 64, 2048, 64), (91, 92, 93, 94)), ((1024, 32, 512, 8), (95, 96, 97, 98))]
    for (M, pad, K, G), seeds in cases:
        x, offs, _ = synthdata.grouped_tokens(M, pad, K, G, seeds=seeds, dtype="bf16")
        xd = x.to("cuda")
        od = torch.from_numpy(offs).to("cuda")
        Ma = M + pad
        outs = []
        for noalloc in (True, False):
            codes = torch.full((Ma, K // 2), 0xA5, dtype=torch.uint8, device="cuda")  # sentinel bytes
            scales = torch.full((Ma, K // 16), 0xA5, dtype=torch.uint8, device="cuda")
            gam = torch.full((G,), -1.0, dtype=torch.float32, device="cuda")
            gsd = torch.full((G,), -1.0, dtype=torch.float32, device="cuda")
            status = torch.zeros(1, dtype=torch.int32, device="cuda")
            if noalloc:
                rc = lib.fos_quantize_grouped_fused_noalloc(_p(xd), 0, Ma, K, _p(od), G, ctypes.byref(cfg),
                                                            _p(codes), _p(scales), _p(gam), _p(gsd), _p(status),
                                                            stream)
            else:
                ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
                rc = lib.fos_quantize_grouped_fused(_p(xd), 0, Ma, K, _p(od), G, ctypes.byref(cfg), _p(codes),
                                                    _p(scales), _p(gam), _p(gsd), _p(ws), _p(status), stream)
            assert rc == 0, lib.fos_last_error()
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            outs.append([t.cpu().numpy() for t in (codes, scales, gam, gsd)])
        for a, b in zip(outs[0], outs[1]):
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8), err_msg=f"{M}x{K} G{G}")
        b = raw_bits(x)
        ga = _group_amaxes(orc, b, "bf16", offs)
        want = orc.quantize_grouped(b, "bf16", offs, ga, recipe="4over6", err_metric="mse", bound=448)
        np.testing.assert_array_equal(outs[0][2].view(np.uint32), ga.view(np.uint32))
        np.testing.assert_array_equal(outs[0][0], want["codes"])
        np.testing.assert_array_equal(outs[0][1], want["scales"])


def test_noalloc_rejects_too_many_groups():
    lib = fos.load_library()
    cfg = fos.config(recipe="4over6")
    x = torch.zeros(64, 32, dtype=torch.bfloat16, device="cuda")
    codes = torch.empty(64, 16, dtype=torch.uint8, device="cuda")
    scales = torch.empty(64, 2, dtype=torch.uint8, device="cuda")
    offs = torch.full((fos.FUSED_MAX_GROUPS + 1,), 64, dtype=torch.int32, device="cuda")
    rc = lib.fos_quantize_grouped_fused_noalloc(_p(x), 0, 64, 32, _p(offs), fos.FUSED_MAX_GROUPS + 1,
                                                ctypes.byref(cfg), _p(codes), _p(scales), None, None, None, None)
    assert rc == 1 and b"exceeds" in lib.fos_last_error()
