"""Pins: the oracle against blocks quantized by hand (tests/golden/hand_blocks.json)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from synthdata import raw_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")
BLOCKS = json.load(open(GOLDEN))["blocks"]


def _val(v):
    return float(v) if not isinstance(v, str) else float(v.replace("nan", "nan"))


def _bf16(vals, shape):
    t = torch.tensor([_val(v) for v in vals], dtype=torch.float32).to(torch.bfloat16).reshape(shape)
    return raw_bits(t)


def _same(a, b):
    if isinstance(b, str) and b == "nan":
        return math.isnan(a)
    return a == b


def _cases():
    for blk in BLOCKS:
        yield pytest.param(blk, "expect", blk["metric"], id=blk["name"] + "-" + blk["metric"])
        if "expect_mae" in blk:
            yield pytest.param(blk, "expect_mae", "mae", id=blk["name"] + "-mae")


@pytest.mark.parametrize("blk,key,metric", list(_cases()))
def test_hand_block(orc, blk, key, metric):
    exp = blk[key]
    if blk["block"] == "1x16":
        x = _bf16(blk["x"], (1, 16))
    else:
        vals = [blk["x_tile"]["rest"]] * 256
        vals[0] = blk["x_tile"]["first"]
        x = _bf16(vals, (16, 16))
    r = orc.quantize(x, "bf16", np.array([blk["amax"]], np.float32), debug=True, recipe="4over6",
                     block=blk["block"], scale_gran="tensor", err_metric=metric, err_prec=blk["prec"],
                     bound=blk["bound"])
    assert int(r["choice"][0]) == exp["choice"]
    assert _same(float(r["err"][0, 0]), exp["err6"])
    assert _same(float(r["err"][0, 1]), exp["err4"])
    if blk["block"] == "1x16":
        assert r["codes"][0].tobytes().hex() == exp["codes"]
        assert r["scales"].tolist() == [[int(exp["scale"], 16)]]
    else:
        assert r["codes"][0].tobytes().hex() == exp["codes_row0"]
        for row in range(1, 16):
            assert r["codes"][row].tobytes().hex() == exp["codes_other"]
        assert r["scales"].reshape(-1).tolist() == [int(exp["scale"], 16)] * 16


def test_hand_block_qdq_negative_zero(orc):
    # the all -0 block dequantizes to bf16 -0 (0x8000) everywhere
    x = _bf16(["-0"] * 16, (1, 16))
    y = orc.qdq(x, "bf16", np.array([2688.0], np.float32), recipe="4over6", err_metric="mse", err_prec="exact")
    assert y.reshape(-1).tolist() == [0x8000] * 16


def test_hand_block_standard_matches_map_to_6(orc):
    # the standard recipe keeps map-to-6 even where four-over-six keeps map-to-4
    x = _bf16([6] + [5] * 15, (1, 16))
    r = orc.quantize(x, "bf16", np.array([2688.0], np.float32), recipe="nvfp4")
    assert r["codes"][0].tobytes().hex() == "6766666666666666"
    assert r["scales"].tolist() == [[0x38]]


def test_hand_zero_tensor_amax(orc):
    # a tensor amax of 0 takes the S_enc = 1 guard: small values round to zero codes
    x = _bf16([0.0] * 15 + [2.0 ** -20], (1, 16))
    r = orc.quantize(x, "bf16", np.array([0.0], np.float32), recipe="4over6", debug=True)
    # a = 2^-20: t6 = RN(2^-20 / 6) << 2^-10, scale 0; t4 = 2^-22, scale 0; codes +0
    assert r["scales"].tolist() == [[0]]
    assert r["codes"][0].tobytes().hex() == "0000000000000000"
    assert r["sdec"].tolist() == [1.0]
