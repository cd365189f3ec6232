"""Four-over-six NVFP4 quantization for AMD MI355X (gfx950).

Python binding of the HIP library ``libfos.so`` (C ABI in ``include/fos.h``).
The functions carry the C entry points' names and only marshal arguments:
PyTorch supplies device memory (outputs are ``torch.empty`` on the input's
device) and the current stream; every step of the quantizer runs in the HIP
kernels. There is no fallback: if the library is missing or the device is not
a gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfos.so")

DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}
RECIPES = {"nvfp4": 0, "4over6": 1}
BLOCKS = {"1x16": 0, "16x16": 1}
GRANS = {"tensor": 0, "row": 1}
METRICS = {"mae": 0, "mse": 1}
PRECS = {"exact": 0, "fp16": 1}
ORDERS = {"tree": 0, "seq": 1}
AMAX_GRANS = {"tensor": 0, "row": 1, "band16": 2}

STATUS_TILE_NONUNIFORM = 1
STATUS_BAD_OFFS = 2
STATUS_BARRIER_TIMEOUT = 4
FUSED_WORKSPACE_BYTES = 16384  # FOS_FUSED_WORKSPACE_BYTES
FUSED_MAX_GROUPS = 256  # FOS_FUSED_MAX_GROUPS


class FosError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fos error {code}: {msg}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [("recipe", ctypes.c_int32), ("block", ctypes.c_int32), ("scale_gran", ctypes.c_int32),
                ("err_metric", ctypes.c_int32), ("err_prec", ctypes.c_int32), ("e4m3_bound", ctypes.c_int32),
                ("err_order", ctypes.c_int32)]


class _Desc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("amax", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SIGS = {
    "fos_abi_version": (_I, []),
    "fos_status_string": (ctypes.c_char_p, [_I]),
    "fos_last_error": (ctypes.c_char_p, []),
    "fos_set_barrier_poll_limit": (_I, [_I]),
    "fos_set_phase_timestamps": (_I, [_P, _I64, _P]),
    "fos_amax": (_I, [_P, _I, _I64, _I64, _I, _P, _P]),
    "fos_quantize": (_I, [_P, _I, _I64, _I64, _P, ctypes.POINTER(_Config), _P, _P, _P, _P, _P]),
    "fos_qdq": (_I, [_P, _I, _I64, _I64, _P, ctypes.POINTER(_Config), _P, _P]),
    "fos_qdq_list": (_I, [_I, _P, _I, ctypes.POINTER(_Config), _P]),
    "fos_qdq_list_fused": (_I, [_I, _P, _I, ctypes.POINTER(_Config), _P, _P, _P, _P]),
    "nvfp4_dequantize": (_I, [_P, _P, _I64, _I64, _P, _I, _I, _P, _P]),
    "fos_quantize_grouped": (_I, [_P, _I, _I64, _I64, _P, _I, _P, ctypes.POINTER(_Config), _P, _P, _P, _P, _P]),
    "fos_quantize_fused": (_I, [_P, _I, _I64, _I64, ctypes.POINTER(_Config), _P, _P, _P, _P, _P, _P, _P]),
    "fos_qdq_fused": (_I, [_P, _I, _I64, _I64, ctypes.POINTER(_Config), _P, _P, _P, _P, _P]),
    "fos_quantize_columnwise": (_I, [_P, _I, _I64, _I64, _P, ctypes.POINTER(_Config), _P, _P, _P, _P]),
    "fos_quantize_grouped_fused": (_I, [_P, _I, _I64, _I64, _P, _I, ctypes.POINTER(_Config), _P, _P, _P, _P, _P, _P,
                                        _P]),
    "fos_quantize_grouped_fused_noalloc": (_I, [_P, _I, _I64, _I64, _P, _I, ctypes.POINTER(_Config), _P, _P, _P, _P,
                                                _P, _P]),
}
EXPORTS = tuple(_SIGS)

_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libfos.so (fails loudly when it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -m nvfp4_adaptive_block_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        lib = load_library()
        raise FosError(rc, lib.fos_last_error().decode())


def config(recipe="4over6", block="1x16", scale_gran="tensor", err_metric="mse", err_prec="exact",
           bound=448, err_order="tree") -> _Config:
    return _Config(RECIPES[recipe], BLOCKS[block], GRANS[scale_gran], METRICS[err_metric], PRECS[err_prec],
                   int(bound), ORDERS[err_order])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(x: torch.Tensor, name: str):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fos_amax(x: torch.Tensor, gran: str = "tensor", out: torch.Tensor | None = None) -> torch.Tensor:
    """NaN-dropping amax per tensor ([1]), per row ([M]) or per 16-row band ([M])."""
    _need(x, "x")
    M, K = x.shape
    if out is None:
        out = torch.empty(1 if gran == "tensor" else M, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(load_library().fos_amax(_ptr(x), DTYPES[x.dtype], M, K, AMAX_GRANS[gran], _ptr(out),
                                       _stream(x.device)))
    return out


def fos_quantize(x: torch.Tensor, amax: torch.Tensor, *, codes=None, scales=None, sdec=None, status=None,
                 **knobs):
    """Quantize x[M, K]. Returns (codes uint8[M, K/2], scales uint8[M, K/16],
    sdec float32[1 or M])."""
    _need(x, "x")
    M, K = x.shape
    cfg = config(**knobs)
    dev = x.device
    if codes is None:
        codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    if sdec is None:
        sdec = torch.empty(M if knobs.get("scale_gran", "tensor") == "row" else 1, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_quantize(_ptr(x), DTYPES[x.dtype], M, K, _ptr(amax), ctypes.byref(cfg),
                                           _ptr(codes), _ptr(scales), _ptr(sdec), _ptr(status), _stream(dev)))
    return codes, scales, sdec


def set_barrier_poll_limit(polls: int) -> int:
    """Polls a fused call's grid barrier makes before giving up (process-wide,
    for calls enqueued from now on); returns the previous limit."""
    prev = load_library().fos_set_barrier_poll_limit(int(polls))
    if prev < 0:
        raise ValueError(f"poll limit must be >= 0, got {polls}")
    return prev


def set_phase_timestamps(buf: torch.Tensor | None) -> int:
    """Diagnostics: the one-read fused kernels enqueued from now on write, per
    wave, four real-time-counter values (start, loads landed, barrier
    released, end) to buf (int64 [waves, 4] on the device); None stops it.
    Returns the counter's rate in kHz."""
    khz = ctypes.c_int(0)
    if buf is None:
        _check(load_library().fos_set_phase_timestamps(None, 0, ctypes.byref(khz)))
    else:
        if buf.dtype != torch.int64 or buf.dim() != 2 or buf.shape[1] != 4 or not buf.is_contiguous():
            raise ValueError("buf must be a contiguous int64 [waves, 4] tensor")
        with torch.cuda.device(buf.device):
            _check(load_library().fos_set_phase_timestamps(ctypes.c_void_p(buf.data_ptr()), buf.shape[0],
                                                           ctypes.byref(khz)))
    return khz.value


def _dev(device) -> torch.device:
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    return dev


# Default workspaces and status words of the fused calls, one of each per
# (device, stream): calls on one stream run one after another and may share
# them; calls on different streams may overlap and must not.
_workspaces: dict = {}
_status_words: dict = {}


def _stream_key(device, stream=None):
    dev = _dev(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return dev, int(s.cuda_stream)


def fused_workspace(device, stream=None) -> torch.Tensor:
    """The zero-initialised workspace the fused calls use on `device` and
    `stream` (default: the device's current stream) when the caller passes
    none."""
    key = _stream_key(device, stream)
    if key not in _workspaces:
        _workspaces[key] = torch.zeros(FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device=key[0])
    return _workspaces[key]


def fused_status_word(device, stream=None) -> torch.Tensor:
    """The device int32 status word the fused calls on `device` and `stream`
    OR their FOS_STATUS_* bits into when the caller passes none. Bits stay
    set until read with fused_status()."""
    key = _stream_key(device, stream)
    if key not in _status_words:
        _status_words[key] = torch.zeros(1, dtype=torch.int32, device=key[0])
    return _status_words[key]


def fused_status(device=None, stream=None, clear: bool = True) -> int:
    """Synchronize `stream` and return the status bits the fused calls on it
    have set since the last read (clearing them unless clear=False)."""
    dev = _dev(device if device is not None else "cuda")
    word = fused_status_word(dev, stream)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    s.synchronize()
    v = int(word.item())
    if clear and v:
        with torch.cuda.stream(s):
            word.zero_()
        s.synchronize()
    return v


def _fused_done(dev, status, own_status: bool, check: bool):
    """After a fused call: with check, synchronize and raise on a barrier
    timeout (the outputs are then incomplete)."""
    if not check:
        return
    torch.cuda.current_stream(dev).synchronize()
    v = int(status.item())
    if own_status and v:
        status.zero_()
        torch.cuda.current_stream(dev).synchronize()
    if v & STATUS_BARRIER_TIMEOUT:
        raise FosError(-1, "fused call: the grid barrier timed out; outputs are incomplete "
                           "(another long-running kernel held part of the device)")


def fos_quantize_fused(x: torch.Tensor, *, codes=None, scales=None, amax=None, sdec=None, status=None,
                       workspace=None, check=False, **knobs):
    """Amax (per tensor, or per row with scale_gran="row") and quantize in
    one launch. Returns (codes, scales, amax float32[1 or M], sdec float32[1
    or M]). Without `workspace` / `status` the current stream's own are used
    (fused_workspace, fused_status_word); with check=True the call
    synchronizes and raises FosError if the grid barrier timed out."""
    _need(x, "x")
    M, K = x.shape
    cfg = config(**knobs)
    dev = x.device
    n_amax = M if knobs.get("scale_gran", "tensor") == "row" else 1
    if codes is None:
        codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    if amax is None:
        amax = torch.empty(n_amax, dtype=torch.float32, device=dev)
    if sdec is None:
        sdec = torch.empty(n_amax, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = fused_workspace(dev)
    own = status is None
    if own:
        status = fused_status_word(dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_quantize_fused(_ptr(x), DTYPES[x.dtype], M, K, ctypes.byref(cfg), _ptr(codes),
                                                 _ptr(scales), _ptr(amax), _ptr(sdec), _ptr(workspace),
                                                 _ptr(status), _stream(dev)))
    _fused_done(dev, status, own, check)
    return codes, scales, amax, sdec


def fos_qdq_fused(x: torch.Tensor, *, out=None, amax=None, status=None, workspace=None, check=False, **knobs):
    """Per-tensor amax and fused quantize-dequantize in one launch (two when
    the tensor does not fit on chip). Returns (y, amax float32[1]).
    `workspace`, `status` and `check` as for fos_quantize_fused."""
    _need(x, "x")
    M, K = x.shape
    cfg = config(**knobs)
    dev = x.device
    y = torch.empty_like(x) if out is None else out
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = fused_workspace(dev)
    own = status is None
    if own:
        status = fused_status_word(dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_qdq_fused(_ptr(x), DTYPES[x.dtype], M, K, ctypes.byref(cfg), _ptr(y), _ptr(amax),
                                            _ptr(workspace), _ptr(status), _stream(dev)))
    _fused_done(dev, status, own, check)
    return y, amax


def fos_quantize_columnwise(x: torch.Tensor, amax: torch.Tensor, *, codes=None, scales=None, sdec=None, **knobs):
    """Quantize the transpose of x[M, K] without materialising it. Returns
    (codes uint8[K, M/2], scales uint8[K, M/16], sdec float32[1])."""
    _need(x, "x")
    M, K = x.shape
    cfg = config(**knobs)
    dev = x.device
    if codes is None:
        codes = torch.empty(K, M // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(K, M // 16, dtype=torch.uint8, device=dev)
    if sdec is None:
        sdec = torch.empty(1, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_quantize_columnwise(_ptr(x), DTYPES[x.dtype], M, K, _ptr(amax), ctypes.byref(cfg),
                                                      _ptr(codes), _ptr(scales), _ptr(sdec), _stream(dev)))
    return codes, scales, sdec


def fos_qdq(x: torch.Tensor, amax: torch.Tensor, *, out=None, **knobs) -> torch.Tensor:
    """Fused quantize-dequantize: y has x's dtype and shape."""
    _need(x, "x")
    M, K = x.shape
    cfg = config(**knobs)
    y = torch.empty_like(x) if out is None else out
    with torch.cuda.device(x.device):
        _check(load_library().fos_qdq(_ptr(x), DTYPES[x.dtype], M, K, _ptr(amax), ctypes.byref(cfg), _ptr(y),
                                      _stream(x.device)))
    return y


def fos_qdq_list(xs: Sequence[torch.Tensor], amaxes: Sequence[torch.Tensor], *, outs=None, **knobs):
    """Fused quantize-dequantize over a list of rank-2 tensors of one dtype."""
    if len(xs) != len(amaxes):
        raise ValueError("xs and amaxes differ in length")
    if not xs:
        return []
    dev = xs[0].device
    ys = [torch.empty_like(x) for x in xs] if outs is None else list(outs)
    descs = (_Desc * len(xs))()
    for i, (x, a, y) in enumerate(zip(xs, amaxes, ys)):
        _need(x, f"xs[{i}]")
        if x.dtype != xs[0].dtype or x.device != dev:
            raise ValueError("all tensors of a list share one dtype and device")
        descs[i] = _Desc(x.data_ptr(), y.data_ptr(), a.data_ptr(), x.shape[0], x.shape[1])
    cfg = config(**knobs)
    with torch.cuda.device(dev):
        _check(load_library().fos_qdq_list(len(xs), ctypes.cast(descs, ctypes.c_void_p), DTYPES[xs[0].dtype],
                                           ctypes.byref(cfg), _stream(dev)))
    return ys


def fos_qdq_list_fused(xs: Sequence[torch.Tensor], *, outs=None, amax=None, workspace=None, status=None,
                       check=False, **knobs):
    """Every tensor's amax and the fused quantize-dequantize of the list in one
    launch. Returns (ys, amax float32[n]). `workspace`, `status` and `check`
    as for fos_quantize_fused."""
    if not xs:
        return [], None
    dev = xs[0].device
    ys = [torch.empty_like(x) for x in xs] if outs is None else list(outs)
    if amax is None:
        amax = torch.empty(len(xs), dtype=torch.float32, device=dev)
    descs = (_Desc * len(xs))()
    for i, (x, y) in enumerate(zip(xs, ys)):
        _need(x, f"xs[{i}]")
        if x.dtype != xs[0].dtype or x.device != dev:
            raise ValueError("all tensors of a list share one dtype and device")
        descs[i] = _Desc(x.data_ptr(), y.data_ptr(), None, x.shape[0], x.shape[1])
    cfg = config(**knobs)
    if workspace is None:
        workspace = fused_workspace(dev)
    own = status is None
    if own:
        status = fused_status_word(dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_qdq_list_fused(len(xs), ctypes.cast(descs, ctypes.c_void_p), DTYPES[xs[0].dtype],
                                                 ctypes.byref(cfg), _ptr(amax), _ptr(workspace), _ptr(status),
                                                 _stream(dev)))
    _fused_done(dev, status, own, check)
    return ys, amax


def nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, sdec: torch.Tensor, scale_gran: str = "tensor",
                     out_dtype: torch.dtype = torch.bfloat16, out=None) -> torch.Tensor:
    """Standard NVFP4 decode of codes[M, K/2] and scales[M, K/16]."""
    _need(codes, "codes")
    M, K = codes.shape[0], codes.shape[1] * 2
    y = torch.empty(M, K, dtype=out_dtype, device=codes.device) if out is None else out
    with torch.cuda.device(codes.device):
        _check(load_library().nvfp4_dequantize(_ptr(codes), _ptr(scales), M, K, _ptr(sdec), GRANS[scale_gran],
                                               DTYPES[out_dtype], _ptr(y), _stream(codes.device)))
    return y


def fos_quantize_grouped(x: torch.Tensor, offs: torch.Tensor, group_amax: torch.Tensor, *, codes=None, scales=None,
                         group_sdec=None, status=None, **knobs):
    """Quantize a packed token tensor of G groups (cumulative end offsets
    ``offs``) with per-group amaxes in one launch. Returns (codes, scales,
    group_sdec)."""
    _need(x, "x")
    M, K = x.shape
    dev = x.device
    G = offs.numel()
    cfg = config(**knobs)
    if codes is None:
        codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    if group_sdec is None:
        group_sdec = torch.empty(G, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_quantize_grouped(_ptr(x), DTYPES[x.dtype], M, K, _ptr(offs), G, _ptr(group_amax),
                                                   ctypes.byref(cfg), _ptr(codes), _ptr(scales), _ptr(group_sdec),
                                                   _ptr(status), _stream(dev)))
    return codes, scales, group_sdec


def fos_quantize_grouped_fused(x: torch.Tensor, offs: torch.Tensor, *, codes=None, scales=None, group_amax=None,
                               group_sdec=None, status=None, workspace=None, check=False, **knobs):
    """Group amaxes and the grouped quantize in one launch. Returns (codes,
    scales, group_amax float32[G], group_sdec float32[G]). `workspace`,
    `status` and `check` as for fos_quantize_fused."""
    _need(x, "x")
    M, K = x.shape
    dev = x.device
    G = offs.numel()
    cfg = config(**knobs)
    if codes is None:
        codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    if group_amax is None:
        group_amax = torch.empty(G, dtype=torch.float32, device=dev)
    if group_sdec is None:
        group_sdec = torch.empty(G, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = fused_workspace(dev)
    own = status is None
    if own:
        status = fused_status_word(dev)
    with torch.cuda.device(dev):
        _check(load_library().fos_quantize_grouped_fused(_ptr(x), DTYPES[x.dtype], M, K, _ptr(offs), G,
                                                         ctypes.byref(cfg), _ptr(codes), _ptr(scales),
                                                         _ptr(group_amax), _ptr(group_sdec), _ptr(workspace),
                                                         _ptr(status), _stream(dev)))
    _fused_done(dev, status, own, check)
    return codes, scales, group_amax, group_sdec


def fos_quantize_grouped_fused_noalloc(x: torch.Tensor, offs: torch.Tensor, *, codes, scales, group_amax,
                                       group_sdec=None, status=None, **knobs):
    """fos_quantize_grouped_fused with the library-held workspace (the C call
    allocates nothing). The caller passes every output buffer. Calls on
    different streams of one device must not overlap."""
    _need(x, "x")
    M, K = x.shape
    dev = x.device
    cfg = config(**knobs)
    with torch.cuda.device(dev):
        _check(load_library().fos_quantize_grouped_fused_noalloc(_ptr(x), DTYPES[x.dtype], M, K, _ptr(offs),
                                                                 offs.numel(), ctypes.byref(cfg), _ptr(codes),
                                                                 _ptr(scales), _ptr(group_amax), _ptr(group_sdec),
                                                                 _ptr(status), _stream(dev)))
    return codes, scales, group_amax, group_sdec
