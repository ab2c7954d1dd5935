"""One variant's delta on disk: the packed signs and alpha of each of its
matrices, in the byte layout the delta cache copies (delta_layout), behind a
small header.

The pages keep each variant as its scale and 1-bit sign matrix and load it on
a cache miss (section "Altyapı ayrıntıları", the cold-start paragraph); the
packed layout of the compression is that storage format.  A file here is the
header, padded to `align` bytes, then the blob exactly as delta_layout lays
it out, so a load reads it straight into page-locked memory for
DeltaCache.attach with no reformatting.

Header (little-endian):
    0  4s   magic b"BDLT"
    4  u32  version (1)
    8  u32  alpha mode (0 per matrix, 1 per row)
   12  u32  number of matrices n
   16  u32  align (the layout's alignment and the header's size unit)
   20  u32  header bytes (a multiple of align)
   24  u64  payload bytes (delta_layout's total for the shapes)
   32  u32  CRC-32 of the payload
   36  u32  CRC-32 of the header bytes with this field zero
   40  n x (u64 d_out, u64 d_in)
then zero bytes up to the header size.
"""

from __future__ import annotations

import os
import struct
import zlib

import torch

from .bitdelta import ALPHA_PER_MATRIX, ALPHA_PER_ROW, delta_layout, delta_views

MAGIC = b"BDLT"
VERSION = 1
MAX_MATRICES = 1 << 16  # bounds the header a reader accepts (about 1 MiB)
_FIXED = struct.Struct("<4sIIIIIQII")
_SHAPE = struct.Struct("<QQ")
_ALIGN = 256


def _check_shapes(shapes, alpha_mode: int):
    if alpha_mode not in (ALPHA_PER_MATRIX, ALPHA_PER_ROW):
        raise ValueError(f"alpha mode {alpha_mode} is neither per matrix nor per row")
    shapes = [(int(o), int(i)) for o, i in shapes]
    if not shapes:
        raise ValueError("a delta holds at least one matrix")
    for d_out, d_in in shapes:
        if d_out < 1 or d_in < 64 or d_in % 64:
            raise ValueError(f"shape ({d_out}, {d_in}): d_out >= 1 and d_in a positive "
                             "multiple of 64")
    return shapes


def _crc(data, crc: int = 0) -> int:
    # zlib.crc32 takes any buffer; 1 GiB pieces keep its length argument in range
    mv = memoryview(data).cast("B")
    step = 1 << 30
    for i in range(0, len(mv), step):
        crc = zlib.crc32(mv[i:i + step], crc)
    return crc & 0xFFFFFFFF


def _header(shapes, alpha_mode: int, payload: int, payload_crc: int) -> bytes:
    body = b"".join(_SHAPE.pack(o, i) for o, i in shapes)
    size = -(-(_FIXED.size + len(body)) // _ALIGN) * _ALIGN
    head = bytearray(size)
    _FIXED.pack_into(head, 0, MAGIC, VERSION, alpha_mode, len(shapes), _ALIGN, size, payload,
                     payload_crc, 0)
    head[_FIXED.size:_FIXED.size + len(body)] = body
    struct.pack_into("<I", head, 36, _crc(head))
    return bytes(head)


def delta_blob(pieces, shapes, alpha_mode: int, pin_memory: bool = True) -> torch.Tensor:
    """A host uint8 blob laid out by delta_layout from one variant's
    [(packed, alpha), ...] (int64 [d_out, d_in/64] and float32 tensors, on
    any device), page-locked unless pin_memory is False."""
    shapes = _check_shapes(shapes, alpha_mode)
    if len(shapes) > MAX_MATRICES:
        raise ValueError(f"at most {MAX_MATRICES} matrices per delta")
    if len(pieces) != len(shapes):
        raise ValueError(f"{len(pieces)} (packed, alpha) pairs for {len(shapes)} shapes")
    _, total = delta_layout(shapes, alpha_mode)
    blob = torch.zeros(total, dtype=torch.uint8, pin_memory=pin_memory)
    for (hp, ha), (p, a), (d_out, d_in) in zip(delta_views(blob, shapes, alpha_mode), pieces,
                                               shapes):
        if p.dtype != torch.int64 or p.numel() != d_out * d_in // 64:
            raise ValueError(f"packed signs of ({d_out}, {d_in}) must be int64 with "
                             f"{d_out * d_in // 64} words")
        if a.dtype != torch.float32 or a.numel() != ha.numel():
            raise ValueError(f"alpha of ({d_out}, {d_in}) must be float32 with {ha.numel()} "
                             "values")
        hp.copy_(p.reshape(hp.shape))
        ha.copy_(a.reshape(-1))
    return blob


def save_delta(path, blob: torch.Tensor, shapes, alpha_mode: int) -> int:
    """Write one variant's delta (a uint8 blob in delta_layout order, host or
    device) to path; returns the file's size in bytes."""
    shapes = _check_shapes(shapes, alpha_mode)
    if len(shapes) > MAX_MATRICES:
        raise ValueError(f"at most {MAX_MATRICES} matrices per delta")
    _, total = delta_layout(shapes, alpha_mode)
    if blob.dtype != torch.uint8 or blob.dim() != 1 or blob.numel() != total:
        raise ValueError(f"the blob must be a 1-D uint8 tensor of {total} bytes for these shapes")
    host = blob.cpu() if blob.device.type != "cpu" else blob
    data = host.contiguous().numpy()
    head = _header(shapes, alpha_mode, total, _crc(data))
    with open(path, "wb") as f:
        f.write(head)
        f.write(memoryview(data))
    return len(head) + total


def read_delta_header(path):
    """(shapes, alpha mode, header bytes, payload bytes, payload CRC-32) of a
    delta file, after checking the header."""
    with open(path, "rb") as f:
        fixed = f.read(_FIXED.size)
        if len(fixed) < _FIXED.size:
            raise ValueError(f"{path}: too short for a delta file header")
        magic, version, mode, n, align, hsize, payload, pcrc, hcrc = _FIXED.unpack(fixed)
        if magic != MAGIC:
            raise ValueError(f"{path}: not a delta file (magic {magic!r})")
        if version != VERSION:
            raise ValueError(f"{path}: delta file version {version}, this reader knows {VERSION}")
        if not 1 <= n <= MAX_MATRICES:
            raise ValueError(f"{path}: {n} matrices in the header (1 .. {MAX_MATRICES})")
        need = -(-(_FIXED.size + n * _SHAPE.size) // _ALIGN) * _ALIGN
        if align != _ALIGN or hsize != need:
            raise ValueError(f"{path}: header size {hsize} or alignment {align} is invalid")
        rest = f.read(hsize - _FIXED.size)
        if len(rest) < hsize - _FIXED.size:
            raise ValueError(f"{path}: truncated header")
    head = bytearray(fixed + rest)
    struct.pack_into("<I", head, 36, 0)
    if _crc(head) != hcrc:
        raise ValueError(f"{path}: header checksum mismatch")
    shapes = [_SHAPE.unpack_from(head, _FIXED.size + _SHAPE.size * k) for k in range(n)]
    shapes = _check_shapes(shapes, mode)
    _, total = delta_layout(shapes, mode)
    if payload != total:
        raise ValueError(f"{path}: payload of {payload} bytes, the shapes lay out {total}")
    return shapes, mode, hsize, payload, pcrc


def load_delta(path, pin_memory: bool = True, verify: bool = True):
    """Read a delta file into a host uint8 blob (page-locked unless
    pin_memory is False) ready for DeltaCache.attach and delta_views.
    Returns (blob, shapes, alpha mode).  verify checks the payload's CRC-32
    (about a gigabyte per second on one host thread)."""
    shapes, mode, hsize, payload, pcrc = read_delta_header(path)
    if os.path.getsize(path) != hsize + payload:
        raise ValueError(f"{path}: {os.path.getsize(path)} bytes, the header announces "
                         f"{hsize + payload}")
    blob = torch.empty(payload, dtype=torch.uint8, pin_memory=pin_memory)
    view = memoryview(blob.numpy())
    with open(path, "rb", buffering=0) as f:
        f.seek(hsize)
        got = 0
        while got < payload:
            n = f.readinto(view[got:])
            if not n:
                raise ValueError(f"{path}: truncated payload")
            got += n
    if verify and _crc(view) != pcrc:
        raise ValueError(f"{path}: payload checksum mismatch")
    return blob, shapes, mode
