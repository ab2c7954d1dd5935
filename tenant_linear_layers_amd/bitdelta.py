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
    10: "BITDELTA_ERR_CACHE",
}

# Delta cache request outcomes and variant states (include/bitdelta.h).
CACHE_HIT, CACHE_QUEUED, CACHE_LOAD, CACHE_FULL = 0, 1, 2, 3
CACHE_ABSENT, CACHE_LOADING, CACHE_RESIDENT = 0, 1, 2

EXPORTS = (
    "bitdelta_compress_workspace_size",
    "bitdelta_compress",
    "bitdelta_compress_noalloc",
    "bitdelta_linear",
    "bitdelta_linear_multi",
    "bitdelta_reconstruct",
    "bitdelta_status_string",
    "bitdelta_ratio_to_f32_bits",
    "bitdelta_cache_create",
    "bitdelta_cache_destroy",
    "bitdelta_cache_request",
    "bitdelta_cache_loaded",
    "bitdelta_cache_release",
    "bitdelta_cache_state",
    "bitdelta_cache_attach",
    "bitdelta_cache_acquire",
    "bitdelta_cache_poll",
    "bitdelta_router_create",
    "bitdelta_router_destroy",
    "bitdelta_router_submit",
    "bitdelta_router_next_batch",
    "bitdelta_router_complete",
    "bitdelta_router_pending",
    "bitdelta_monosoup_workspace_size",
    "bitdelta_monosoup_merge",
    "bitdelta_probe_stream_read",
    "bitdelta_probe_mfma_bf16",
    "bitdelta_probe_decode_loads",
)

MONOSOUP_MAX_RANK = 32
MONOSOUP_MAX_CHECKPOINTS = 64
MONOSOUP_MAX_POWER_ITERS = 64


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
    L.bitdelta_compress_noalloc.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
    L.bitdelta_compress_noalloc.restype = i32
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
    pi32, pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    L.bitdelta_cache_create.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i64,
                                        ctypes.POINTER(vp)]
    L.bitdelta_cache_create.restype = i32
    L.bitdelta_cache_destroy.argtypes = [vp]
    L.bitdelta_cache_destroy.restype = None
    L.bitdelta_cache_request.argtypes = [vp, ctypes.c_int32, pi32, pi32, pi32]
    L.bitdelta_cache_request.restype = i32
    L.bitdelta_cache_loaded.argtypes = [vp, ctypes.c_int32]
    L.bitdelta_cache_loaded.restype = i32
    L.bitdelta_cache_release.argtypes = [vp, ctypes.c_int32, vp]
    L.bitdelta_cache_release.restype = i32
    L.bitdelta_cache_state.argtypes = [vp, ctypes.c_int32, pi32, pi32, pi64]
    L.bitdelta_cache_state.restype = i32
    L.bitdelta_cache_attach.argtypes = [vp, vp, sz, vp, vp]
    L.bitdelta_cache_attach.restype = i32
    L.bitdelta_cache_acquire.argtypes = [vp, ctypes.c_int32, vp, vp, pi32, ctypes.POINTER(vp),
                                         pi32]
    L.bitdelta_cache_acquire.restype = i32
    L.bitdelta_cache_poll.argtypes = [vp, pi32]
    L.bitdelta_cache_poll.restype = i32
    L.bitdelta_router_create.argtypes = [vp, ctypes.POINTER(vp)]
    L.bitdelta_router_create.restype = i32
    L.bitdelta_router_destroy.argtypes = [vp]
    L.bitdelta_router_destroy.restype = None
    L.bitdelta_router_submit.argtypes = [vp, i64, ctypes.c_int32]
    L.bitdelta_router_submit.restype = i32
    L.bitdelta_router_next_batch.argtypes = [vp, ctypes.c_int32, vp, pi64, pi32, pi32, pi32]
    L.bitdelta_router_next_batch.restype = i32
    L.bitdelta_router_complete.argtypes = [vp, ctypes.c_int32, pi32, vp]
    L.bitdelta_router_complete.restype = i32
    L.bitdelta_router_pending.argtypes = [vp, pi32]
    L.bitdelta_router_pending.restype = i32
    L.bitdelta_monosoup_workspace_size.argtypes = [i64, i64, ctypes.c_int32, ctypes.c_int32]
    L.bitdelta_monosoup_workspace_size.restype = sz
    L.bitdelta_monosoup_merge.argtypes = [vp, ctypes.c_int32, vp, i64, i64, ctypes.c_int32,
                                          ctypes.c_int32, vp, vp, vp, vp, sz, vp]
    L.bitdelta_monosoup_merge.restype = i32
    L.bitdelta_probe_stream_read.argtypes = [vp, sz, ctypes.c_int32, vp, vp]
    L.bitdelta_probe_stream_read.restype = i32
    L.bitdelta_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
    L.bitdelta_probe_mfma_bf16.restype = i32
    L.bitdelta_probe_decode_loads.argtypes = [vp, vp, vp, ctypes.c_int32, vp, vp]
    L.bitdelta_probe_decode_loads.restype = i32
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


def compress_noalloc(w_ft: torch.Tensor, w_base: torch.Tensor, alpha_mode: int, packed: torch.Tensor,
                     alpha: torch.Tensor, stream=None):
    """compress into caller tensors through bitdelta_compress_noalloc (no
    workspace, nothing allocated by the library or here)."""
    _need(w_base, "w_base", torch.bfloat16)
    dev = w_base.device
    _need(w_ft, "w_ft", torch.bfloat16, dev)
    if w_base.dim() != 2 or w_ft.shape != w_base.shape:
        raise ValueError("w_ft and w_base must be 2-D and of one shape")
    d_out, d_in = w_base.shape
    _need(packed, "packed", torch.int64, dev)
    _need(alpha, "alpha", torch.float32, dev)
    _signs_and_scale(packed, alpha, d_out, d_in, alpha_mode)
    with _on(dev):
        st = lib().bitdelta_compress_noalloc(_ptr(w_ft), _ptr(w_base), d_out, d_in, alpha_mode,
                                             _ptr(packed), _ptr(alpha), _stream(stream))
    _check(st, "bitdelta_compress_noalloc")
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


# ------------------------------------------------------------------ delta cache
def delta_layout(shapes, alpha_mode: int, align: int = 256):
    """Byte layout of one variant's delta for a list of matrix shapes
    [(d_out, d_in), ...]: each matrix's packed signs (d_out*d_in/8 bytes),
    then its alpha (4*d_out or 4 bytes), every piece starting on `align`
    bytes.  Returns ([(packed_offset, alpha_offset), ...], total_bytes)."""
    off, out = 0, []
    for d_out, d_in in shapes:
        p = off
        off = -(-(p + d_out * d_in // 8) // align) * align
        a = off
        off = -(-(a + 4 * (d_out if alpha_mode == ALPHA_PER_ROW else 1)) // align) * align
        out.append((p, a))
    return out, off


def delta_views(buf: torch.Tensor, shapes, alpha_mode: int):
    """(packed int64 [d_out, d_in/64], alpha float32) views of each matrix's
    piece of a uint8 buffer laid out by delta_layout (host or device)."""
    if buf.dtype != torch.uint8 or buf.dim() != 1:
        raise TypeError("buf must be a 1-D uint8 tensor")
    offs, total = delta_layout(shapes, alpha_mode)
    if buf.numel() < total:
        raise ValueError(f"buf holds {buf.numel()} bytes, the layout needs {total}")
    views = []
    for (d_out, d_in), (p, a) in zip(shapes, offs):
        na = d_out if alpha_mode == ALPHA_PER_ROW else 1
        packed = buf[p:p + d_out * d_in // 8].view(torch.int64).view(d_out, d_in // 64)
        alpha = buf[a:a + 4 * na].view(torch.float32)
        views.append((packed, alpha))
    return views


class DeltaCache:
    """A libbitdelta delta cache (bitdelta_cache_*): the request-rate pinned
    LRU policy over device slots, and, once attach() has given it slots and
    per-variant host sources, the host-to-device loads that fill them."""

    def __init__(self, n_variants: int, n_slots: int, n_pinned: int = 0,
                 halve_every: int = 0):
        h = ctypes.c_void_p()
        _check(lib().bitdelta_cache_create(n_variants, n_slots, n_pinned, halve_every,
                                           ctypes.byref(h)), "bitdelta_cache_create")
        self._h = h
        self.n_variants, self.n_slots = n_variants, n_slots
        self._slots = None
        self._sources = None
        self._slot_of_ptr = {}

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().bitdelta_cache_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def _triple(self):
        return ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()

    def request(self, variant: int):
        """Policy only: (action, slot, evicted) of one request."""
        a, s, e = self._triple()
        _check(lib().bitdelta_cache_request(self._h, variant, ctypes.byref(a), ctypes.byref(s),
                                            ctypes.byref(e)), "bitdelta_cache_request")
        return a.value, s.value, e.value

    def loaded(self, variant: int) -> None:
        _check(lib().bitdelta_cache_loaded(self._h, variant), "bitdelta_cache_loaded")

    def release(self, variant: int, stream=None) -> None:
        st = _stream(stream) if self._slots is not None else ctypes.c_void_p(None)
        _check(lib().bitdelta_cache_release(self._h, variant, st), "bitdelta_cache_release")

    def state(self, variant: int):
        """(state, slot, rate) of a variant."""
        st, sl, r = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
        _check(lib().bitdelta_cache_state(self._h, variant, ctypes.byref(st), ctypes.byref(sl),
                                          ctypes.byref(r)), "bitdelta_cache_state")
        return st.value, sl.value, r.value

    def attach(self, slots, sources) -> None:
        """slots: n_slots device uint8 tensors of one size; sources: n_variants
        host uint8 tensors (page-locked for asynchronous copies), each no
        larger than a slot.  Both lists are kept alive by the cache."""
        if len(slots) != self.n_slots or len(sources) != self.n_variants:
            raise ValueError("one tensor per slot and one source per variant")
        nbytes = slots[0].numel()
        for t in slots:
            _need(t, "slot", torch.uint8, slots[0].device)
            _size(t, "slot", nbytes)
        for t in sources:
            if t.dtype != torch.uint8 or t.is_cuda or not t.is_contiguous():
                raise ValueError("sources must be contiguous host uint8 tensors")
        sarr = (ctypes.c_void_p * len(slots))(*[t.data_ptr() for t in slots])
        varr = (ctypes.c_void_p * len(sources))(*[t.data_ptr() for t in sources])
        barr = (ctypes.c_size_t * len(sources))(*[t.numel() for t in sources])
        with _on(slots[0].device):
            st = lib().bitdelta_cache_attach(self._h, ctypes.cast(sarr, ctypes.c_void_p), nbytes,
                                             ctypes.cast(varr, ctypes.c_void_p),
                                             ctypes.cast(barr, ctypes.c_void_p))
        _check(st, "bitdelta_cache_attach")
        self._slots, self._sources = list(slots), list(sources)
        self._slot_of_ptr = {t.data_ptr(): i for i, t in enumerate(slots)}

    def acquire(self, variant: int, copy_stream, use_stream=None):
        """(action, slot tensor or None, evicted) of one request that moves the
        bytes: after it, work on use_stream reads the variant's delta."""
        if self._slots is None:
            raise RuntimeError("attach() the cache's memory first")
        a, e = ctypes.c_int32(), ctypes.c_int32()
        ptr = ctypes.c_void_p()
        with _on(self._slots[0].device):
            st = lib().bitdelta_cache_acquire(self._h, variant, _stream(copy_stream),
                                              _stream(use_stream), ctypes.byref(a),
                                              ctypes.byref(ptr), ctypes.byref(e))
        _check(st, "bitdelta_cache_acquire")
        slot = None if not ptr.value else self._slots[self._slot_of_ptr[ptr.value]]
        return a.value, slot, e.value

    def poll(self) -> int:
        n = ctypes.c_int32()
        _check(lib().bitdelta_cache_poll(self._h, ctypes.byref(n)), "bitdelta_cache_poll")
        return n.value


class Router:
    """A libbitdelta router (bitdelta_router_*) over a DeltaCache: decode
    batches of ready requests in arrival order; with the cache's memory
    attached, registering a request starts its load on the copy stream."""

    def __init__(self, cache: DeltaCache):
        h = ctypes.c_void_p()
        _check(lib().bitdelta_router_create(cache._h, ctypes.byref(h)), "bitdelta_router_create")
        self._h = h
        self.cache = cache          # kept alive: the cache must outlive the router

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().bitdelta_router_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def submit(self, request_id: int, variant: int) -> None:
        _check(lib().bitdelta_router_submit(self._h, request_id, variant), "bitdelta_router_submit")

    def next_batch(self, max_batch: int, copy_stream=None):
        """[(request id, variant, slot)] of the next batch (slot -1 for the base)."""
        ids = (ctypes.c_int64 * max(max_batch, 1))()
        vs = (ctypes.c_int32 * max(max_batch, 1))()
        ss = (ctypes.c_int32 * max(max_batch, 1))()
        n = ctypes.c_int32()
        attached = self.cache._slots is not None
        cs = _stream(copy_stream) if attached else ctypes.c_void_p(None)
        if attached:
            with _on(self.cache._slots[0].device):
                st = lib().bitdelta_router_next_batch(self._h, max_batch, cs, ids, vs, ss,
                                                      ctypes.byref(n))
        else:
            st = lib().bitdelta_router_next_batch(self._h, max_batch, cs, ids, vs, ss,
                                                  ctypes.byref(n))
        _check(st, "bitdelta_router_next_batch")
        return [(int(ids[i]), int(vs[i]), int(ss[i])) for i in range(n.value)]

    def complete(self, batch, use_stream=None) -> None:
        vs = (ctypes.c_int32 * max(len(batch), 1))(*[b[1] for b in batch])
        st_ = _stream(use_stream) if self.cache._slots is not None else ctypes.c_void_p(None)
        _check(lib().bitdelta_router_complete(self._h, len(batch), vs, st_),
               "bitdelta_router_complete")

    def pending(self) -> int:
        n = ctypes.c_int32()
        _check(lib().bitdelta_router_pending(self._h, ctypes.byref(n)), "bitdelta_router_pending")
        return n.value


# ------------------------------------------------------------------ MonoSoup
def monosoup_workspace_size(d_out: int, d_in: int, k: int, rank: int) -> int:
    return int(lib().bitdelta_monosoup_workspace_size(d_out, d_in, k, rank))


def monosoup_merge(w_fts, w_base: torch.Tensor, rank: int, power_iters: int,
                   omega: torch.Tensor, want_tau: bool = False, out=None, workspace=None,
                   stream=None):
    """(merged bf16 [d_out, d_in], mean of the rank-r truncations float32 or
    None) for k checkpoints w_fts of the base w_base; omega float32
    [d_in, rank] is the Gaussian start of the orthogonal iteration."""
    _need(w_base, "w_base", torch.bfloat16)
    dev = w_base.device
    if w_base.dim() != 2:
        raise ValueError("w_base must be 2-D")
    d_out, d_in = w_base.shape
    for w in w_fts:
        _need(w, "w_ft", torch.bfloat16, dev)
        if w.shape != w_base.shape:
            raise ValueError("every checkpoint must have the base's shape")
    _need(omega, "omega", torch.float32, dev)
    _size(omega, "omega", d_in * rank)
    k = len(w_fts)
    if out is None:
        out = torch.empty_like(w_base)
    _need(out, "out", torch.bfloat16, dev)
    _size(out, "out", d_out * d_in)
    tau = torch.empty((d_out, d_in), dtype=torch.float32, device=dev) if want_tau else None
    need = monosoup_workspace_size(d_out, d_in, k, rank)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * max(k, 1))(*[w.data_ptr() for w in w_fts])
    with _on(dev):
        st = lib().bitdelta_monosoup_merge(ctypes.cast(arr, ctypes.c_void_p), k, _ptr(w_base),
                                           d_out, d_in, rank, power_iters, _ptr(omega), _ptr(out),
                                           _ptr(tau), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "bitdelta_monosoup_merge")
    return out, tau


# ------------------------------------------------------------------ calibration
def probe_stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None):
    """One plain read of every byte of src (device, 16-byte multiple) by
    `workgroups` workgroups; sink: device tensor of at least 1024 bytes."""
    if not src.is_cuda or not src.is_contiguous() or not sink.is_cuda:
        raise ValueError("src and sink must be contiguous device tensors")
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("sink must hold at least 1024 bytes")
    nbytes = src.numel() * src.element_size()
    with _on(src.device):
        st = lib().bitdelta_probe_stream_read(_ptr(src), nbytes, workgroups, _ptr(sink),
                                              _stream(stream))
    _check(st, "bitdelta_probe_stream_read")


def probe_mfma_bf16(workgroups: int, iters: int, sink: torch.Tensor, stream=None) -> int:
    """Back-to-back bf16 matrix-core instructions; returns the flops issued."""
    if not sink.is_cuda or sink.numel() * sink.element_size() < 1024:
        raise ValueError("sink must be a device tensor of at least 1024 bytes")
    with _on(sink.device):
        st = lib().bitdelta_probe_mfma_bf16(workgroups, iters, _ptr(sink), _stream(stream))
    _check(st, "bitdelta_probe_mfma_bf16")
    return 1048576 * workgroups * iters


def probe_decode_loads(w: torch.Tensor, signs: torch.Tensor, x: torch.Tensor, mode: int,
                       sink: torch.Tensor, stream=None):
    """The single-variant decode's loads on a 4096 x 4096 bf16 matrix without
    its arithmetic (mode 0..5, see include/bitdelta.h); w: [4096, 4096] bf16,
    signs: at least 2 MiB, x: at least 8 KiB, sink: at least 1024 bytes, all
    contiguous device tensors."""
    for t in (w, signs, x, sink):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all arguments must be contiguous device tensors")
    if w.dtype != torch.bfloat16 or tuple(w.shape) != (4096, 4096):
        raise ValueError("w must be a [4096, 4096] bf16 tensor")
    nb = lambda t: t.numel() * t.element_size()
    if nb(signs) < (1 << 21) or nb(x) < 8192 or nb(sink) < 1024:
        raise ValueError("signs, x and sink must hold 2 MiB, 8 KiB and 1 KiB")
    with _on(w.device):
        st = lib().bitdelta_probe_decode_loads(_ptr(w), _ptr(signs), _ptr(x), mode, _ptr(sink),
                                               _stream(stream))
    _check(st, "bitdelta_probe_decode_loads")
