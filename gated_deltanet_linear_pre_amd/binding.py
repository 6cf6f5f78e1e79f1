"""Thin ctypes binding of libgdn.so (include/gdn.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, the stream defaults
to torch's current stream, and a non-zero status raises GdnError.  Every step
of the path runs in the library's HIP kernels; there is no fallback.  If
libgdn.so is missing, lib() raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")
HEADER = os.path.join(HERE, "..", "include", "gdn.h")

GDN_F32, GDN_F16 = 0, 1
DTYPE_CODE = {"f32": GDN_F32, "f16": GDN_F16}

STATUS = {0: "GDN_OK", -1: "GDN_E_NULL", -2: "GDN_E_SHAPE", -3: "GDN_E_ALIGN",
          -4: "GDN_E_WORKSPACE", -5: "GDN_E_DTYPE", -6: "GDN_E_LAUNCH", -7: "GDN_E_TOO_LARGE"}


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {gdn_status_str(status)}")


class gdn_shape(ctypes.Structure):
    _fields_ = [("hk", ctypes.c_int32), ("hv", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("n_seq", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("total_T", ctypes.c_int64), ("max_T", ctypes.c_int64),
                ("eps_l2", ctypes.c_float), ("eps_rms", ctypes.c_float)]


def make_shape(hk: int, hv: int, n_seq: int, total_T: int, max_T: int, io: str = "f16",
               out: str = "f16", eps_l2: float = 1e-6, eps_rms: float = 1e-6,
               dk: int = 128, dv: int = 128) -> gdn_shape:
    return gdn_shape(hk, hv, dk, dv, n_seq, DTYPE_CODE.get(io, io), DTYPE_CODE.get(out, out), 0,
                     total_T, max_T, eps_l2, eps_rms)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run gated_deltanet_linear_pre_amd.build "
                               "(or __graft_entry__.build()) first; there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        SP = ctypes.POINTER(gdn_shape)
        L.gdn_abi_version.restype = I
        L.gdn_abi_version.argtypes = []
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_status_str.argtypes = [I]
        L.gdn_pre.restype = I
        L.gdn_pre.argtypes = [SP] + [P] * 14
        L.gdn_scan.restype = I
        L.gdn_scan.argtypes = [SP] + [P] * 9 + [S, P]
        L.gdn_scan_workspace_bytes.restype = S
        L.gdn_scan_workspace_bytes.argtypes = [SP]
        L.gdn_post.restype = I
        L.gdn_post.argtypes = [SP] + [P] * 5
        L.gdn_prefill_workspace_bytes.restype = S
        L.gdn_prefill_workspace_bytes.argtypes = [SP]
        L.gdn_prefill_layer.restype = I
        L.gdn_prefill_layer.argtypes = [SP] + [P] * 13 + [S, P]
        L.gdn_prefill_layer_noalloc.restype = I
        L.gdn_prefill_layer_noalloc.argtypes = [SP] + [P] * 13
        L.gdn_step.restype = I
        L.gdn_step.argtypes = [SP] + [P] * 13
        _lib = L
    return _lib


def declared_symbols() -> list[str]:
    """Function names include/gdn.h declares (for the export check)."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(gdn_\w+)\s*\(", text, re.M)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise GdnError(fn, status)


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def gdn_status_str(status: int) -> str:
    return lib().gdn_status_str(status).decode()


def gdn_pre(shape, cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist, qn, kn, vc, g, beta,
            stream=None, check=True) -> int:
    st = lib().gdn_pre(ctypes.byref(shape), *map(_ptr, (cu_seqlens, qkv, conv_w, a, b, A_log,
                                                           dt_bias, hist, qn, kn, vc, g, beta)),
                       _stream(stream))
    if check:
        _check("gdn_pre", st)
    return st


def gdn_scan_workspace_bytes(shape) -> int:
    return int(lib().gdn_scan_workspace_bytes(ctypes.byref(shape)))


def gdn_scan(shape, cu_seqlens, qn, kn, vc, g, beta, state, o, workspace, workspace_bytes=None,
             stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gdn_scan(ctypes.byref(shape), *map(_ptr, (cu_seqlens, qn, kn, vc, g, beta, state, o,
                                                            workspace)),
                        int(workspace_bytes), _stream(stream))
    if check:
        _check("gdn_scan", st)
    return st


def gdn_post(shape, o, z, gamma, y, stream=None, check=True) -> int:
    st = lib().gdn_post(ctypes.byref(shape), *map(_ptr, (o, z, gamma, y)), _stream(stream))
    if check:
        _check("gdn_post", st)
    return st


def gdn_prefill_workspace_bytes(shape) -> int:
    return int(lib().gdn_prefill_workspace_bytes(ctypes.byref(shape)))


def gdn_prefill_layer(shape, cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist, state,
                      y, workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gdn_prefill_layer(
        ctypes.byref(shape), *map(_ptr, (cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma,
                                         hist, state, y, workspace)),
        int(workspace_bytes), _stream(stream))
    if check:
        _check("gdn_prefill_layer", st)
    return st


def gdn_prefill_layer_noalloc(shape, cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist,
                              state, y, stream=None, check=True) -> int:
    st = lib().gdn_prefill_layer_noalloc(
        ctypes.byref(shape), *map(_ptr, (cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma,
                                         hist, state, y)),
        _stream(stream))
    if check:
        _check("gdn_prefill_layer_noalloc", st)
    return st


def gdn_step(shape, qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist, state, y, stream=None,
             check=True, hist_out=None) -> int:
    st = lib().gdn_step(ctypes.byref(shape), *map(_ptr, (qkv, conv_w, a, b, A_log, dt_bias, z,
                                                            gamma, hist, hist_out, state, y)),
                        _stream(stream))
    if check:
        _check("gdn_step", st)
    return st
