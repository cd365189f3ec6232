"""CPU oracle for the four-over-six NVFP4 quantizer (ctypes wrapper).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``nvfp4_adaptive_block_amd``) never imports it and shares no code with it.

The arithmetic lives in ``fos_oracle.c`` (plain C, binary32, OpenMP over block
rows); see the header of that file for the passages each step follows. This
module only marshals numpy arrays. High-precision tensors travel as their raw
bits: ``uint16`` arrays for bfloat16 and float16, ``float32`` for fp32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fos_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2}
RECIPES = {"nvfp4": 0, "4over6": 1, "map4": 2}
BLOCKS = {"1x16": 0, "16x16": 1}
GRANS = {"tensor": 0, "row": 1}
METRICS = {"mae": 0, "mse": 1}
PRECS = {"exact": 0, "fp16": 1}
ORDERS = {"tree": 0, "seq": 1}
AMAX_MODES = {"tensor": 0, "row": 1, "band16": 2}

STATUS_TILE_NONUNIFORM = 1
STATUS_BAD_OFFS = 2

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True, out: str | None = None, src: str | None = None) -> str:
    """Compile the oracle with gcc into ``liboracle.so`` (or ``out``)."""
    out = out or _LIB_PATH
    src = src or _SRC
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, "-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("recipe", ctypes.c_int32), ("block", ctypes.c_int32),
                ("scale_gran", ctypes.c_int32), ("err_metric", ctypes.c_int32),
                ("err_prec", ctypes.c_int32), ("e4m3_bound", ctypes.c_int32),
                ("err_order", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "oracle_e2m1_value": (ctypes.c_float, [ctypes.c_int]),
    "oracle_e4m3_value": (ctypes.c_float, [ctypes.c_int]),
    "oracle_e2m1_rne_sat": (ctypes.c_int, [ctypes.c_float]),
    "oracle_e4m3_rne_sat": (ctypes.c_int, [ctypes.c_float]),
    "oracle_f16_bits_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "oracle_f32_to_f16_rne": (ctypes.c_uint16, [ctypes.c_float]),
    "oracle_f32_to_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
    "oracle_bf16_bits_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "oracle_e2m1_rne_sat_array": (None, [_P, _I64, _P]),
    "oracle_e4m3_rne_sat_array": (None, [_P, _I64, _P]),
    "oracle_f32_to_f16_rne_array": (None, [_P, _I64, _P]),
    "oracle_f32_to_bf16_rne_array": (None, [_P, _I64, _P]),
    "oracle_global_encode_scale": (ctypes.c_float, [ctypes.c_float, ctypes.c_int]),
    "oracle_global_decode_scale": (ctypes.c_float, [ctypes.c_float, ctypes.c_int]),
    "oracle_global_scales_array": (None, [_P, _I64, ctypes.c_int, _P, _P]),
    "oracle_tree16": (ctypes.c_float, [_P]),
    "oracle_seq16": (ctypes.c_float, [_P]),
    "oracle_amax": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, ctypes.c_int, _P]),
    "oracle_quantize": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, ctypes.POINTER(_Cfg),
                                       _P, _P, _P, _P, _P, _P, _P]),
    "oracle_qdq": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, ctypes.POINTER(_Cfg), _P]),
    "oracle_dequantize": (ctypes.c_int, [_P, _P, _I64, _I64, _P, ctypes.c_int, ctypes.c_int, _P]),
    "oracle_quantize_grouped": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, ctypes.c_int, _P,
                                               ctypes.POINTER(_Cfg), _P, _P, _P, _P]),
    "oracle_num_threads": (ctypes.c_int, []),
}

_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    path = path or _LIB_PATH
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != _LIB_PATH:
            raise FileNotFoundError(path)
        build(force=False)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib_cache[path] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cfg(recipe="4over6", block="1x16", scale_gran="tensor", err_metric="mse", err_prec="exact",
         bound=448, err_order="tree") -> _Cfg:
    return _Cfg(RECIPES[recipe], BLOCKS[block], GRANS[scale_gran], METRICS[err_metric],
                PRECS[err_prec], int(bound), ORDERS[err_order])


def _check_x(x, dtype):
    x = np.ascontiguousarray(x)
    want = np.float32 if dtype == "fp32" else np.uint16
    if x.dtype != want or x.ndim != 2:
        raise TypeError(f"oracle input for {dtype} must be a 2-D {np.dtype(want).name} array")
    return x


class Oracle:
    """Thin marshalling layer over one loaded oracle library."""

    def __init__(self, path: str | None = None):
        self.lib = load(path)

    # ---- element formats -------------------------------------------------
    def e2m1_value(self, code: int) -> float:
        return self.lib.oracle_e2m1_value(code)

    def e4m3_value(self, code: int) -> float:
        return self.lib.oracle_e4m3_value(code)

    def e2m1_rne_sat(self, v) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.empty(v.shape, np.uint8)
        self.lib.oracle_e2m1_rne_sat_array(_ptr(v), v.size, _ptr(out))
        return out

    def e4m3_rne_sat(self, t) -> np.ndarray:
        t = np.ascontiguousarray(t, dtype=np.float32)
        out = np.empty(t.shape, np.uint8)
        self.lib.oracle_e4m3_rne_sat_array(_ptr(t), t.size, _ptr(out))
        return out

    def f32_to_f16_bits(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_f32_to_f16_rne_array(_ptr(x), x.size, _ptr(out))
        return out

    def f32_to_bf16_bits(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_f32_to_bf16_rne_array(_ptr(x), x.size, _ptr(out))
        return out

    def global_encode_scale(self, amax: float, bound: int) -> float:
        return self.lib.oracle_global_encode_scale(amax, bound)

    def global_decode_scale(self, amax: float, bound: int) -> float:
        return self.lib.oracle_global_decode_scale(amax, bound)

    def global_scales(self, amax, bound: int):
        """(S_enc, S_dec) arrays of an array of amaxes."""
        a = np.ascontiguousarray(amax, dtype=np.float32)
        enc = np.empty(a.shape, np.float32)
        dec = np.empty(a.shape, np.float32)
        self.lib.oracle_global_scales_array(_ptr(a), a.size, bound, _ptr(enc), _ptr(dec))
        return enc, dec

    def seq16(self, u) -> float:
        u = np.ascontiguousarray(u, dtype=np.float32)
        assert u.size == 16
        return self.lib.oracle_seq16(_ptr(u))

    def tree16(self, u) -> float:
        u = np.ascontiguousarray(u, dtype=np.float32)
        assert u.size == 16
        return self.lib.oracle_tree16(_ptr(u))

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    # ---- tensors ---------------------------------------------------------
    def amax(self, x, dtype: str, mode: str = "tensor") -> np.ndarray:
        x = _check_x(x, dtype)
        M, K = x.shape
        out = np.zeros(1 if mode == "tensor" else M, np.float32)
        rc = self.lib.oracle_amax(_ptr(x), DTYPES[dtype], M, K, AMAX_MODES[mode], _ptr(out))
        if rc:
            raise ValueError(f"oracle_amax rejected the arguments ({rc})")
        return out

    def quantize(self, x, dtype: str, amax, *, debug: bool = False, **knobs) -> dict:
        x = _check_x(x, dtype)
        M, K = x.shape
        cfg = _cfg(**knobs)
        amax = np.ascontiguousarray(amax, dtype=np.float32).reshape(-1)
        codes = np.zeros((M, K // 2), np.uint8)
        scales = np.zeros((M, K // 16), np.uint8)
        sdec = np.zeros(amax.size, np.float32)
        status = np.zeros(1, np.int32)
        bh = 16 if knobs.get("block", "1x16") == "16x16" else 1
        nblk = (M // bh) * (K // 16)
        xhat = np.zeros((M, K), np.float32) if debug else None
        choice = np.zeros(nblk, np.uint8) if debug else None
        err = np.zeros((nblk, 2), np.float32) if debug else None
        rc = self.lib.oracle_quantize(_ptr(x), DTYPES[dtype], M, K, _ptr(amax), ctypes.byref(cfg),
                                      _ptr(codes), _ptr(scales), _ptr(sdec), _ptr(xhat), _ptr(choice),
                                      _ptr(err), _ptr(status))
        if rc:
            raise ValueError(f"oracle_quantize rejected the arguments ({rc})")
        out = {"codes": codes, "scales": scales, "sdec": sdec, "status": int(status[0])}
        if debug:
            out.update(xhat=xhat, choice=choice, err=err)
        return out

    def qdq(self, x, dtype: str, amax, **knobs) -> np.ndarray:
        x = _check_x(x, dtype)
        M, K = x.shape
        cfg = _cfg(**knobs)
        amax = np.ascontiguousarray(amax, dtype=np.float32).reshape(-1)
        y = np.zeros_like(x)
        rc = self.lib.oracle_qdq(_ptr(x), DTYPES[dtype], M, K, _ptr(amax), ctypes.byref(cfg), _ptr(y))
        if rc:
            raise ValueError(f"oracle_qdq rejected the arguments ({rc})")
        return y

    def dequantize(self, codes, scales, sdec, scale_gran: str, out_dtype: str) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        sdec = np.ascontiguousarray(sdec, dtype=np.float32).reshape(-1)
        M, K = codes.shape[0], codes.shape[1] * 2
        y = np.zeros((M, K), np.float32 if out_dtype == "fp32" else np.uint16)
        rc = self.lib.oracle_dequantize(_ptr(codes), _ptr(scales), M, K, _ptr(sdec), GRANS[scale_gran],
                                        DTYPES[out_dtype], _ptr(y))
        if rc:
            raise ValueError(f"oracle_dequantize rejected the arguments ({rc})")
        return y

    def quantize_grouped(self, x, dtype: str, offs, group_amax, **knobs) -> dict:
        x = _check_x(x, dtype)
        M_alloc, K = x.shape
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        group_amax = np.ascontiguousarray(group_amax, dtype=np.float32)
        G = offs.size
        cfg = _cfg(**knobs)
        codes = np.zeros((M_alloc, K // 2), np.uint8)
        scales = np.zeros((M_alloc, K // 16), np.uint8)
        gsdec = np.zeros(G, np.float32)
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_quantize_grouped(_ptr(x), DTYPES[dtype], M_alloc, K, _ptr(offs), G,
                                              _ptr(group_amax), ctypes.byref(cfg), _ptr(codes),
                                              _ptr(scales), _ptr(gsdec), _ptr(status))
        if rc:
            raise ValueError(f"oracle_quantize_grouped rejected the arguments ({rc})")
        return {"codes": codes, "scales": scales, "group_sdec": gsdec, "status": int(status[0])}


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from this directory's source."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
