"""CPU pin of the division by 6 that the kernels use for the map-to-6 block
scale (pytorch/ao PR "Add the four-over-six grouped GEMM and dispatcher
wiring", recipe commit: the map-to-6 candidate; wolfcomos/ao PR, description:
correctly rounded FP32 division is rounding-critical). The formula
RN(a * RN(1/6)) corrected by one fused multiply-add of the exact remainder
is checked on every non-negative binary32 against IEEE RN(a / 6), in
binary32 with hardware FMAs (tests/div6_formula.c). It is exact for every
finite a >= 2^-125. Below that some quotients are subnormal, and at +inf
the remainder is inf - inf, and it is not: the device helper divides for
those inputs instead (which tests/test_gpu_primitives.py checks on the
device).
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _cpu_has_fma():
    try:
        return " fma " in " " + open("/proc/cpuinfo").read().replace("\n", " ") + " "
    except OSError:
        return False


@pytest.mark.skipif(not _cpu_has_fma(), reason="the check uses the CPU's fused multiply-add")
def test_div6_formula_is_correctly_rounded_above_2_pow_minus_125(tmp_path):
    exe = str(tmp_path / "div6_formula")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
                    os.path.join(HERE, "div6_formula.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    above, below, inf, checked = (int(v) for v in out)
    assert checked == 0x7F800001
    assert above == 0, f"{above} finite inputs >= 2^-125 are not correctly rounded"
    # the two input ranges the helper sends to the division instead
    assert below > 0, "the formula was expected to miss some subnormal quotients"
    assert inf == 1, "the formula was expected to give NaN at +inf"
