"""Thin ctypes binding of libbitdelta (include/bitdelta.h).

Argument marshalling only: every step of the BitDelta path runs in the HIP
kernels of libbitdelta.so.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is not built or a call fails,
an exception is raised.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitdelta.so")

ALPHA_PER_MATRIX = 0
ALPHA_PER_ROW = 1
MAX_VARIANTS = 64

STATUS_NAMES = {
    0: "BITDELTA_OK",
    1: "BITDELTA_ERR_NULL",
    2: "BITDELTA_ERR_SHAPE",
    3: "BITDELTA_ERR_ALIGN",
    4: "BITDELTA_ERR_MODE",
    5: "BITDELTA_ERR_VARIANTS",
    6: "BITDELTA_ERR_WORKSPACE",
    7: "BITDELTA_ERR_HIP",
    8: "BITDELTA_ERR_DEVICE",
    9: "BITDELTA_ERR_OVERLAP",
}

EXPORTS = (
    "bitdelta_compress_workspace_size",
    "bitdelta_compress",
    "bitdelta_linear",
    "bitdelta_linear_multi",
    "bitdelta_reconstruct",
    "bitdelta_status_string",
    "bitdelta_ratio_to_f32_bits",
)


class BitDeltaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library with argument types declared.  torch is imported
    first so that the library binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m tenant_linear_layers_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.bitdelta_compress_workspace_size.argtypes = [i64, i64, i32]
    L.bitdelta_compress_workspace_size.restype = sz
    L.bitdelta_compress.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, sz, vp]
    L.bitdelta_compress.restype = i32
    L.bitdelta_linear.argtypes = [vp, i64, vp, vp, vp, i32, i64, i64, vp, vp]
    L.bitdelta_linear.restype = i32
    L.bitdelta_linear_multi.argtypes = [vp, i64, vp, vp, ctypes.c_int32, vp, vp, i32, i64, i64,
                                        vp, vp]
    L.bitdelta_linear_multi.restype = i32
    L.bitdelta_reconstruct.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp]
    L.bitdelta_reconstruct.restype = i32
    L.bitdelta_status_string.argtypes = [i32]
    L.bitdelta_status_string.restype = ctypes.c_char_p
    L.bitdelta_ratio_to_f32_bits.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
    L.bitdelta_ratio_to_f32_bits.restype = ctypes.c_uint32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().bitdelta_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise BitDeltaError(status, where)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _on(dev: torch.device):
    """Make dev the current HIP device for the call (a no-op when it is)."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(None if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _size(t: torch.Tensor, name: str, n: int):
    """The library reads or writes exactly n elements through t's pointer."""
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()} ({tuple(t.shape)})")


def _signs_and_scale(packed, alpha, d_out: int, d_in: int, alpha_mode: int, pname="packed",
                     aname="alpha"):
    if d_in % 64 == 0:  # other widths are rejected by the library itself
        _size(packed, pname, d_out * (d_in // 64))
    if alpha_mode in (ALPHA_PER_MATRIX, ALPHA_PER_ROW):
        _size(alpha, aname, d_out if alpha_mode == ALPHA_PER_ROW else 1)


def ratio_to_f32_bits(s: int, n: int) -> int:
    """Host copy of the scale's final rounding: float32 bits of s / (n * 2^48)."""
    return int(lib().bitdelta_ratio_to_f32_bits((s >> 64) & (2**64 - 1), s & (2**64 - 1), n))


def compress_workspace_size(d_out: int, d_in: int, alpha_mode: int) -> int:
    return int(lib().bitdelta_compress_workspace_size(d_out, d_in, alpha_mode))


def compress(w_ft: torch.Tensor, w_base: torch.Tensor, alpha_mode: int, packed=None,
             alpha=None, workspace=None, stream=None):
    """(packed int64 [d_out, d_in/64] holding the uint64 words, alpha float32
    [1] or [d_out]) for one matrix."""
    _need(w_base, "w_base", torch.bfloat16)
    _need(w_ft, "w_ft", torch.bfloat16, w_base.device)
    if w_base.dim() != 2 or w_ft.shape != w_base.shape:
        raise ValueError("w_ft and w_base must be 2-D and of one shape")
    d_out, d_in = w_base.shape
    dev = w_base.device
    if packed is None:
        packed = torch.empty((d_out, max(d_in // 64, 1)), dtype=torch.int64, device=dev)
    if alpha is None:
        alpha = torch.empty((d_out if alpha_mode == ALPHA_PER_ROW else 1,), dtype=torch.float32,
                            device=dev)
    _need(packed, "packed", torch.int64, dev)
    _need(alpha, "alpha", torch.float32, dev)
    _signs_and_scale(packed, alpha, d_out, d_in, alpha_mode)
    need = compress_workspace_size(d_out, d_in, alpha_mode)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with _on(dev):
        st = lib().bitdelta_compress(_ptr(w_ft), _ptr(w_base), d_out, d_in, alpha_mode,
                                     _ptr(packed), _ptr(alpha), _ptr(workspace), ws_bytes,
                                     _stream(stream))
    _check(st, "bitdelta_compress")
    return packed, alpha


def linear(x: torch.Tensor, w_base: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor,
           alpha_mode: int, y=None, stream=None) -> torch.Tensor:
    """y = x (W_base + alpha sign(Delta))^T; x [..., d_in] bf16 -> y [..., d_out] bf16."""
    _need(w_base, "w_base", torch.bfloat16)
    dev = w_base.device
    _need(x, "x", torch.bfloat16, dev)
    _need(packed, "packed", torch.int64, dev)
    _need(alpha, "alpha", torch.float32, dev)
    d_out, d_in = w_base.shape
    if x.shape[-1] != d_in:
        raise ValueError("x's last dimension must equal d_in")
    lead = x.shape[:-1]
    m = x.numel() // d_in
    _signs_and_scale(packed, alpha, d_out, d_in, alpha_mode)
    if y is None:
        y = torch.empty((*lead, d_out), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev)
    _size(y, "y", m * d_out)
    with _on(dev):
        st = lib().bitdelta_linear(_ptr(x), m, _ptr(w_base), _ptr(packed), _ptr(alpha),
                                   alpha_mode, d_out, d_in, _ptr(y), _stream(stream))
    _check(st, "bitdelta_linear")
    return y


def linear_multi(x: torch.Tensor, variant_ids: torch.Tensor, w_base: torch.Tensor,
                 packed_list, alpha_list, alpha_mode: int, y=None, stream=None) -> torch.Tensor:
    """Mixed-variant batch: token m uses variant variant_ids[m] (-1 = base only)."""
    _need(w_base, "w_base", torch.bfloat16)
    dev = w_base.device
    _need(x, "x", torch.bfloat16, dev)
    _need(variant_ids, "variant_ids", torch.int32, dev)
    d_out, d_in = w_base.shape
    m = x.numel() // d_in
    if x.shape[-1] != d_in or variant_ids.numel() != m:
        raise ValueError("x must be [..., d_in] with one variant id per token")
    nv = len(packed_list)
    if nv != len(alpha_list):
        raise ValueError("one alpha per packed variant")
    for p, a in zip(packed_list, alpha_list):
        _need(p, "packed", torch.int64, dev)
        _need(a, "alpha", torch.float32, dev)
        _signs_and_scale(p, a, d_out, d_in, alpha_mode)
    if y is None:
        y = torch.empty((*x.shape[:-1], d_out), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev)
    _size(y, "y", m * d_out)
    parr = (ctypes.c_void_p * max(nv, 1))(*[p.data_ptr() for p in packed_list])
    aarr = (ctypes.c_void_p * max(nv, 1))(*[a.data_ptr() for a in alpha_list])
    with _on(dev):
        st = lib().bitdelta_linear_multi(_ptr(x), m, _ptr(variant_ids), _ptr(w_base), nv,
                                         ctypes.cast(parr, ctypes.c_void_p),
                                         ctypes.cast(aarr, ctypes.c_void_p), alpha_mode, d_out,
                                         d_in, _ptr(y), _stream(stream))
    _check(st, "bitdelta_linear_multi")
    return y


def reconstruct(w_base: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor,
                alpha_mode: int, w_eff=None, stream=None) -> torch.Tensor:
    """W_eff = bf16(W_base + alpha sign(Delta)), bf16 [d_out, d_in] (the unfused path)."""
    _need(w_base, "w_base", torch.bfloat16)
    dev = w_base.device
    _need(packed, "packed", torch.int64, dev)
    _need(alpha, "alpha", torch.float32, dev)
    if w_base.dim() != 2:
        raise ValueError("w_base must be 2-D")
    d_out, d_in = w_base.shape
    _signs_and_scale(packed, alpha, d_out, d_in, alpha_mode)
    if w_eff is None:
        w_eff = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)
    _need(w_eff, "w_eff", torch.bfloat16, dev)
    _size(w_eff, "w_eff", d_out * d_in)
    with _on(dev):
        st = lib().bitdelta_reconstruct(_ptr(w_base), _ptr(packed), _ptr(alpha), alpha_mode,
                                        d_out, d_in, _ptr(w_eff), _stream(stream))
    _check(st, "bitdelta_reconstruct")
    return w_eff
