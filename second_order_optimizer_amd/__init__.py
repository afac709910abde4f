"""Python binding of libkfac.so (include/kfac.h): argument marshalling only.

Every step of the optimizer runs in the library's HIP kernels; this module
only builds the C descriptor structs from tensor pointers, passes the current
HIP stream, and turns status codes into exceptions.  PyTorch is used for
device memory and streams.  There is no fallback: if the shared library is
missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# KFAC_LIBRARY names another build of the same library (the host-sanitized
# one the sanitizer test loads); there is no fallback when it is missing.
LIB_PATH = os.environ.get("KFAC_LIBRARY") or os.path.join(_PKG, "libkfac.so")

KFAC_OK, KFAC_ERR_ARG, KFAC_ERR_DTYPE, KFAC_ERR_ALIGN, KFAC_ERR_WORKSPACE, KFAC_ERR_UNSUPPORTED, KFAC_ERR_HIP = range(7)
LINEAR, CONV2D, BATCHNORM = 0, 1, 2
FACTORS_FULL, FACTORS_PACKED = 0, 1
REFRESH_A, REFRESH_G, REFRESH_BOTH = 1, 2, 3
OPT_RESCALE = 1
WARMUP_LINEAR, WARMUP_GEOMETRIC = 0, 1
F32, BF16 = 0, 1
MODE_FULL, MODE_DIAG = 0, 1
PHASE_FACTORS, PHASE_INVERT, PHASE_UPDATE, PHASE_RESCALE, PHASE_ALL = 1, 2, 4, 8, 15
FLAG_NOT_PD, FLAG_NONFINITE = 1, 2

EXPORTS = ("kfac_workspace_size", "kfac_step_full", "kfac_step_diag", "kfac_step_diag_noalloc", "kfac_read_flags",
           "kfac_schedule_hparams", "kfac_status_string", "kfac_abi_version")
NOALLOC_SCRATCH_BYTES = 32 << 20


class Layer(ctypes.Structure):
    """Mirror of kfac_layer_t."""
    _fields_ = [
        ("kind", ctypes.c_int32), ("has_bias", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
        ("rows", ctypes.c_int64), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("c_in", ctypes.c_int32), ("height", ctypes.c_int32),
        ("width", ctypes.c_int32), ("kh", ctypes.c_int32), ("kw", ctypes.c_int32),
        ("stride", ctypes.c_int32), ("pad", ctypes.c_int32),
        ("factor_layout", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("a", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("grad_w", ctypes.c_void_p), ("grad_b", ctypes.c_void_p),
        ("w", ctypes.c_void_p), ("b", ctypes.c_void_p),
        ("mom_w", ctypes.c_void_p), ("mom_b", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("G", ctypes.c_void_p),
        ("A_inv", ctypes.c_void_p), ("G_inv", ctypes.c_void_p),
        ("F_w", ctypes.c_void_p), ("F_b", ctypes.c_void_p),
        ("dA", ctypes.c_void_p), ("dG", ctypes.c_void_p),
    ]


class HParams(ctypes.Structure):
    """Mirror of kfac_hparams_t."""
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("ema_decay", ctypes.c_float),
                ("damping", ctypes.c_float), ("damping_bn", ctypes.c_float),
                ("rescale_eps", ctypes.c_float), ("refresh", ctypes.c_int32),
                ("phase_mask", ctypes.c_int32), ("options", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Schedule(ctypes.Structure):
    """Mirror of kfac_schedule_t."""
    _fields_ = [("damping_init", ctypes.c_float), ("damping_target", ctypes.c_float),
                ("warmup_steps", ctypes.c_int32), ("warmup_shape", ctypes.c_int32),
                ("bn_damping_scale", ctypes.c_float), ("dense_steps", ctypes.c_int32),
                ("refresh_every_a", ctypes.c_int32), ("refresh_every_g", ctypes.c_int32)]


class KfacError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Loads libkfac.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is missing: build it with "
                                "`python -m second_order_optimizer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kfac_workspace_size.argtypes = [ctypes.POINTER(Layer), i32, i32, ctypes.POINTER(sz)]
    lib.kfac_workspace_size.restype = i32
    for fn in (lib.kfac_step_full, lib.kfac_step_diag):
        fn.argtypes = [ctypes.POINTER(Layer), i32, ctypes.POINTER(HParams), vp, sz, vp]
        fn.restype = i32
    lib.kfac_step_diag_noalloc.argtypes = [ctypes.POINTER(Layer), i32, ctypes.POINTER(HParams), vp, vp]
    lib.kfac_step_diag_noalloc.restype = i32
    lib.kfac_read_flags.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32), i32]
    lib.kfac_read_flags.restype = i32
    lib.kfac_schedule_hparams.argtypes = [ctypes.POINTER(Schedule), ctypes.c_int64, ctypes.POINTER(HParams)]
    lib.kfac_schedule_hparams.restype = i32
    lib.kfac_status_string.argtypes = [i32]
    lib.kfac_status_string.restype = ctypes.c_char_p
    lib.kfac_abi_version.argtypes = []
    lib.kfac_abi_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kfac_status_string(status).decode()


def abi_version() -> int:
    return load().kfac_abi_version()


def _array(layers: Sequence[Layer]):
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L
    return arr


def workspace_size(layers: Sequence[Layer], mode: int) -> int:
    out = ctypes.c_size_t(0)
    st = load().kfac_workspace_size(_array(layers) if layers else None, len(layers), mode, ctypes.byref(out))
    if st != KFAC_OK:
        raise KfacError(st, "kfac_workspace_size")
    return out.value


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def hparams(lr, momentum, weight_decay, ema_decay, damping, refresh=True, phase_mask=0, damping_bn=None,
            rescale_eps=1e-9, options=0) -> HParams:
    """refresh: True (both inverses), False, or KFAC_REFRESH_* bits;
    damping_bn defaults to damping."""
    bits = REFRESH_BOTH if refresh is True else (0 if refresh is False else int(refresh))
    return HParams(lr, momentum, weight_decay, ema_decay, damping, damping if damping_bn is None else damping_bn,
                   rescale_eps, bits, phase_mask, options, 0)


def schedule_hparams(sched: Schedule, step: int, hp: HParams) -> HParams:
    """kfac_schedule_hparams: fills damping, damping_bn and refresh of hp for
    `step` (host only)."""
    st = load().kfac_schedule_hparams(ctypes.byref(sched), step, ctypes.byref(hp))
    if st != KFAC_OK:
        raise KfacError(st, "kfac_schedule_hparams")
    return hp


def step_full(layers, hp: HParams, workspace: int, ws_bytes: int, stream=None) -> None:
    """kfac_step_full; `layers` is a Layer array (see ``layer_array``)."""
    st = load().kfac_step_full(layers, len(layers), ctypes.byref(hp), workspace, ws_bytes, _stream_handle(stream))
    if st != KFAC_OK:
        raise KfacError(st, "kfac_step_full")


def step_diag(layers, hp: HParams, workspace: int, ws_bytes: int, stream=None) -> None:
    """kfac_step_diag; `layers` is a Layer array (see ``layer_array``)."""
    st = load().kfac_step_diag(layers, len(layers), ctypes.byref(hp), workspace, ws_bytes, _stream_handle(stream))
    if st != KFAC_OK:
        raise KfacError(st, "kfac_step_diag")


def step_diag_noalloc(layers, hp: HParams, flags: int, stream=None) -> None:
    """kfac_step_diag_noalloc: `flags` is the device address of a zeroed
    uint32 flag word (no workspace; the library's own scratch array is used)."""
    st = load().kfac_step_diag_noalloc(layers, len(layers), ctypes.byref(hp), flags, _stream_handle(stream))
    if st != KFAC_OK:
        raise KfacError(st, "kfac_step_diag_noalloc")


def read_flags(workspace: int, clear: bool = False, stream=None) -> int:
    out = ctypes.c_uint32(0)
    st = load().kfac_read_flags(workspace, _stream_handle(stream), ctypes.byref(out), int(bool(clear)))
    if st != KFAC_OK:
        raise KfacError(st, "kfac_read_flags")
    return out.value


def layer_array(layers: Sequence[Layer]):
    """A contiguous C array of descriptors (kept by the caller across steps)."""
    return _array(layers)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_layer(kind: int, d_in: int, d_out: int, rows: int, has_bias: bool, *, act_dtype=F32, grad_dtype=F32,
               batch=0, c_in=0, height=0, width=0, k=0, stride=0, pad=0, factor_layout=FACTORS_FULL,
               **tensors) -> Layer:
    """Builds one descriptor; keyword tensors (torch, on the GPU) are taken by
    pointer: a, g, grad_w, grad_b, w, b, mom_w, mom_b, A, G, A_inv, G_inv,
    F_w, F_b, dA, dG.  The caller keeps the tensors alive."""
    L = Layer()
    L.kind, L.has_bias, L.act_dtype, L.grad_dtype = kind, int(has_bias), act_dtype, grad_dtype
    L.rows, L.d_in, L.d_out = rows, d_in, d_out
    L.batch, L.c_in, L.height, L.width = batch, c_in, height, width
    L.kh = L.kw = k
    L.stride, L.pad = stride, pad
    L.factor_layout = factor_layout
    for name, t in tensors.items():
        if not hasattr(L, name):
            raise KeyError(name)
        setattr(L, name, _ptr(t))
    return L
