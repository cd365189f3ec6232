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
    assert lib.fos_abi_version() == 6
    assert lib.fos_status_string(0) == b"ok"
    assert lib.fos_status_string(3) == b"unsupported shape"
    # a shape error is reported before any device is touched
    cfg = fos.config()
    rc = lib.fos_quantize(None, 0, 4, 40, None, ctypes.byref(cfg), None, None, None, None, None)
    assert rc != 0
    # the barrier's poll limit: set, read back through the previous value, restored
    prev = lib.fos_set_barrier_poll_limit(7)
    assert prev == 1 << 20
    assert lib.fos_set_barrier_poll_limit(-1) == -1
    assert lib.fos_set_barrier_poll_limit(prev) == 7


def test_fused_calls_validate_before_touching_a_device():
    """The fused entry points' argument checks run on the host and return
    their error codes before any device call (fake, never-dereferenced
    addresses stand in for device buffers)."""
    lib = fos.load_library()
    P = ctypes.c_void_p
    x, y, ws, a = P(0x10000), P(0x20000), P(0x30000), P(0x40000)
    cfg = fos.config(recipe="4over6")
    tiles = fos.config(recipe="4over6", block="16x16")
    rows = fos.config(recipe="4over6", scale_gran="row")
    # fos_qdq_fused: 1x16 with a per-tensor scale only; y, amax_out and workspace required; 8-byte workspace
    assert lib.fos_qdq_fused(x, 0, 16, 64, ctypes.byref(tiles), y, a, ws, None, None) == 5   # FOS_ERR_CONFIG
    assert lib.fos_qdq_fused(x, 0, 16, 64, ctypes.byref(rows), y, a, ws, None, None) == 5
    assert lib.fos_qdq_fused(x, 0, 16, 40, ctypes.byref(cfg), y, a, ws, None, None) == 3     # FOS_ERR_SHAPE
    assert lib.fos_qdq_fused(x, 0, 16, 64, ctypes.byref(cfg), y, None, ws, None, None) == 1  # amax_out NULL
    assert lib.fos_qdq_fused(x, 0, 16, 64, ctypes.byref(cfg), y, a, None, None, None) == 1   # workspace NULL
    assert lib.fos_qdq_fused(x, 0, 16, 64, ctypes.byref(cfg), y, a, P(0x30004), None, None) == 4  # FOS_ERR_ALIGN
    assert lib.fos_qdq_fused(x, 0, 16, 64, ctypes.byref(cfg), P(0x20008), a, ws, None, None) == 4
    # fos_quantize_fused: 16x16 is rejected; per-row passes the argument checks
    codes, scales = P(0x50000), P(0x60000)
    assert lib.fos_quantize_fused(x, 0, 16, 64, ctypes.byref(tiles), codes, scales, a, None, ws, None, None) == 5
    rc = lib.fos_quantize_fused(x, 0, 16, 64, ctypes.byref(rows), codes, scales, a, None, P(0x30004), None, None)
    assert rc == 4, "per-row is accepted up to the workspace alignment check"


def test_product_package_does_not_reach_the_oracle():
    """The product path imports, includes and links nothing under oracle/."""
    pkg = os.path.join(ROOT, "nvfp4_adaptive_block_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                for bad in ("import oracle", "from oracle", "fos_oracle", "liboracle"):
                    assert bad not in text, (f, bad)
