"""The C-ABI library loads and exports every entry point include/fos.h declares
(CPU only: no compute call is made without a GPU)."""
import ctypes
import os
import re

import nvfp4_adaptive_block_amd as fos

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fos.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("fos_quantize", "fos_qdq", "fos_qdq_list", "nvfp4_dequantize", "fos_quantize_grouped", "fos_amax",
                 "fos_abi_version", "fos_status_string", "fos_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fos.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(fos.EXPORTS)


def test_host_only_calls():
    lib = fos.load_library()
    assert lib.fos_abi_version() == 4
    assert lib.fos_status_string(0) == b"ok"
    assert lib.fos_status_string(3) == b"unsupported shape"
    # a shape error is reported before any device is touched
    cfg = fos.config()
    rc = lib.fos_quantize(None, 0, 4, 40, None, ctypes.byref(cfg), None, None, None, None, None)
    assert rc != 0


def test_product_package_does_not_reach_the_oracle():
    """The product path imports, includes and links nothing under oracle/."""
    pkg = os.path.join(ROOT, "nvfp4_adaptive_block_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                for bad in ("import oracle", "from oracle", "fos_oracle", "liboracle"):
                    assert bad not in text, (f, bad)
