"""Host logic of bench.py (CPU only): the one-GPU contract, the profile
summaries' freshness rule, the kernel descriptions, the step's bytes and the
static occupancy rule."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profile_values_need_the_current_kernel_sources(tmp_path):
    good = tmp_path / "good.txt"
    good.write_text(f"kernel_source_sha256_16 = {bench.kernel_source_hash()}\nhbm_bytes_per_launch = 123.5\n")
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha256_16 = 0000000000000000\nhbm_bytes_per_launch = 123.5\n")
    assert bench.read_profile_value(str(good), "hbm_bytes_per_launch") == 123.5
    assert bench.read_profile_value(str(good), "missing_key") is None
    assert bench.read_profile_value(str(stale), "hbm_bytes_per_launch") is None
    assert bench.read_profile_value(str(tmp_path / "absent.txt"), "hbm_bytes_per_launch") is None


def test_kernel_descriptions():
    d = bench.describe_kernel
    assert d("void fos::k_1x16<1, 0, 1, 1, 0, 0, 0, 0>(fos::Args1x16<1>)") == \
        "1x16 quantize bf16 4over6 mse exact tensor"
    assert d("void fos::k_1x16<48, 1, 1, 0, 1, 1, 0, 1>(fos::Args1x16<48>)") == \
        "1x16 qdq list<48> fp16 4over6 mae fp16err seq tensor"
    assert d("void fos::k_fused_onchip<0, 1, 1, 0, 0, 0>(fos::Args1x16<1>, unsigned int*, float*)") == \
        "fused amax + 1x16 quantize (one read) bf16 4over6 mse exact tensor"
    assert d(bench.HEADLINE_KERNEL) == "1x16 quantize bf16 4over6 mse exact grouped"
    assert d("void fos::k_fused_onchip<1, 1, 0, 1, 0, 1>(fos::Args1x16<1>, unsigned int*, float*)") == \
        "fused amax + 1x16 qdq (one read) fp16 4over6 mae fp16err tensor"
    assert d("void fos::k_fused<0, 1, 1, 0, 0>(fos::Args1x16<1>, unsigned int*, float*)") == \
        "fused amax + 1x16 quantize (two reads) bf16 4over6 mse exact tensor"
    assert d("void fos::k_16x16<2, 1, 1, 0, 1, 0>(fos::Args16x16)").startswith("16x16 quantize fp32 4over6")
    assert "grouped" in d("void fos::k_fused_grouped<0, 1, 1, 0, 0>(fos::Args1x16<1>, unsigned int*, float*)")
    assert d("void fos::k_fused_row<0, 1, 1, 0, 0>(fos::Args1x16<1>, float*)") == \
        "fused row amaxes + 1x16 quantize bf16 4over6 mse exact"
    assert d("void fos::k_colwise<0, 1, 1, 0, 0>(fos::Args16x16)").startswith("columnwise")
    assert d("void fos::k_dequant<0, 0>(unsigned char const*)") == "dequantize to bf16 tensor"
    assert d("some_other_kernel") == ""


def test_step_bytes_of_the_grouped_step():
    # the 65536 data rows are read once (2 B per element); codes and scales
    # are written for all 69632 rows, padding included (0.5625 B per element)
    M, pad, K = 65536, 4096, 7168
    assert bench.STEP_BYTES == M * K * 2 + (M + pad) * K * 9 // 16 == 1220280320
    assert bench.COUNTER_KERNELS[bench.HEADLINE_KERNEL][2] == bench.STEP_BYTES
    # per 1x16 block of the dense activation tensor: 32 B read, codes 8 B, scale 1 B
    blocks = 8192 * 4096 // 16
    for name, (_, _, alg) in bench.COUNTER_KERNELS.items():
        if "8192x4096" in bench.COUNTER_KERNELS[name][0]:
            assert alg == blocks * 41


def test_kernel_resources_need_the_current_kernel_sources(tmp_path):
    name = bench.HEADLINE_KERNEL
    good = tmp_path / "good.txt"
    good.write_text(f"# kernel_source_sha256_16 = {bench.kernel_source_hash()}\n"
                    f"{name} | sgprs=106 vgprs=95 occupancy_waves_per_simd=5\n")
    stale = tmp_path / "stale.txt"
    stale.write_text(f"# kernel_source_sha256_16 = 0000000000000000\n{name} | vgprs=95\n")
    assert bench.kernel_resources(name, str(good)) == {"sgprs": "106", "vgprs": "95", "occupancy_waves_per_simd": "5"}
    assert bench.kernel_resources("void fos::k_other<0>(int)", str(good)) == {}
    assert bench.kernel_resources(name, str(stale)) == {}
