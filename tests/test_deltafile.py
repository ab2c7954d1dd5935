"""Delta files (tenant_linear_layers_amd.deltafile): one variant's packed
signs and alpha behind a small header, the payload in the delta cache's
byte layout.  CPU only: round trips are byte-exact, the header encodes what
its documentation says, and damaged or mismatched files are refused."""

import os
import struct
import zlib

import pytest
import torch

import tenant_linear_layers_amd as T

SHAPES = [(256, 512), (64, 128), (3, 64)]


def pieces(shapes, mode, seed):
    g = torch.Generator().manual_seed(seed)
    out = []
    for d_out, d_in in shapes:
        p = torch.randint(-2 ** 62, 2 ** 62, (d_out, d_in // 64), generator=g, dtype=torch.int64)
        a = torch.rand(d_out if mode == T.ALPHA_PER_ROW else 1, generator=g)
        out.append((p, a))
    return out


@pytest.mark.parametrize("mode", [T.ALPHA_PER_MATRIX, T.ALPHA_PER_ROW])
def test_round_trip_is_byte_exact(tmp_path, mode):
    pc = pieces(SHAPES, mode, 1 + mode)
    blob = T.delta_blob(pc, SHAPES, mode, pin_memory=False)
    path = tmp_path / "v.bdlt"
    n = T.save_delta(path, blob, SHAPES, mode)
    assert n == os.path.getsize(path)
    back, shapes, m = T.load_delta(path, pin_memory=False)
    assert shapes == SHAPES and m == mode
    assert torch.equal(back, blob)
    # the loaded blob is the cache layout: its views are the variant's tensors
    for (p, a), (lp, la) in zip(pc, T.delta_views(back, SHAPES, mode)):
        assert torch.equal(lp, p) and torch.equal(la, a)


def test_header_layout(tmp_path):
    """The fields at the documented offsets, the header padded to 256 bytes,
    the payload right after it."""
    mode = T.ALPHA_PER_ROW
    blob = T.delta_blob(pieces(SHAPES, mode, 5), SHAPES, mode, pin_memory=False)
    path = tmp_path / "v.bdlt"
    T.save_delta(path, blob, SHAPES, mode)
    raw = path.read_bytes()
    magic, ver, m, n, align, hsize, payload, pcrc, hcrc = struct.unpack_from("<4sIIIIIQII", raw)
    assert (magic, ver, m, n, align) == (b"BDLT", 1, mode, len(SHAPES), 256)
    assert hsize == 256 and payload == blob.numel() == len(raw) - hsize
    assert [struct.unpack_from("<QQ", raw, 40 + 16 * k) for k in range(n)] == SHAPES
    assert raw[40 + 16 * n:hsize] == bytes(hsize - 40 - 16 * n)
    assert pcrc == zlib.crc32(raw[hsize:])
    head = bytearray(raw[:hsize])
    head[36:40] = bytes(4)
    assert hcrc == zlib.crc32(head)
    assert raw[hsize:] == blob.numpy().tobytes()
    assert T.read_delta_header(path) == (SHAPES, mode, hsize, payload, pcrc)


def test_many_matrices_header_spans_blocks(tmp_path):
    shapes = [(16 + k, 64 * (1 + k % 3)) for k in range(20)]  # 40 + 320 bytes of header
    mode = T.ALPHA_PER_MATRIX
    blob = T.delta_blob(pieces(shapes, mode, 9), shapes, mode, pin_memory=False)
    path = tmp_path / "v.bdlt"
    T.save_delta(path, blob, shapes, mode)
    shp, m, hsize, payload, _ = T.read_delta_header(path)
    assert shp == shapes and hsize == 512 and payload == blob.numel()
    assert torch.equal(T.load_delta(path, pin_memory=False)[0], blob)


def _saved(tmp_path):
    mode = T.ALPHA_PER_ROW
    blob = T.delta_blob(pieces(SHAPES, mode, 3), SHAPES, mode, pin_memory=False)
    path = tmp_path / "v.bdlt"
    T.save_delta(path, blob, SHAPES, mode)
    return path, bytearray(path.read_bytes())


def _write(path, data):
    path.write_bytes(bytes(data))
    return path


def test_damaged_payload_is_refused(tmp_path):
    path, raw = _saved(tmp_path)
    raw[256 + 1000] ^= 0x10
    _write(path, raw)
    with pytest.raises(ValueError, match="payload checksum"):
        T.load_delta(path, pin_memory=False)
    blob, _, _ = T.load_delta(path, pin_memory=False, verify=False)  # unchecked read still works
    assert blob[1000].item() == raw[256 + 1000]


@pytest.mark.parametrize("offset,match", [(0, "not a delta file"), (4, "version"),
                                          (12, "header"), (44, "header checksum"),
                                          (24, "header checksum")])
def test_damaged_header_is_refused(tmp_path, offset, match):
    path, raw = _saved(tmp_path)
    raw[offset] ^= 0x01
    _write(path, raw)
    with pytest.raises(ValueError, match=match):
        T.load_delta(path, pin_memory=False)


def test_oversized_header_fields_are_refused_before_reading(tmp_path):
    """A header announcing a huge matrix count or header size is refused
    from its fixed fields, before anything that size is read."""
    path, raw = _saved(tmp_path)
    big = bytearray(raw)
    struct.pack_into("<I", big, 12, 1 << 30)          # matrices
    _write(path, big)
    with pytest.raises(ValueError, match="matrices in the header"):
        T.load_delta(path, pin_memory=False)
    big = bytearray(raw)
    struct.pack_into("<I", big, 20, (1 << 31) - 256)  # header bytes
    _write(path, big)
    with pytest.raises(ValueError, match="header size"):
        T.load_delta(path, pin_memory=False)


def test_truncated_files_are_refused(tmp_path):
    path, raw = _saved(tmp_path)
    for cut in (10, 100, len(raw) - 1):
        _write(path, raw[:cut])
        with pytest.raises(ValueError):
            T.load_delta(path, pin_memory=False)
    _write(path, raw + b"\0")
    with pytest.raises(ValueError, match="announces"):
        T.load_delta(path, pin_memory=False)


def test_arguments_are_checked(tmp_path):
    mode = T.ALPHA_PER_ROW
    pc = pieces(SHAPES, mode, 4)
    with pytest.raises(ValueError):
        T.delta_blob(pc[:2], SHAPES, mode, pin_memory=False)
    with pytest.raises(ValueError):
        T.delta_blob(pc, SHAPES, T.ALPHA_PER_MATRIX, pin_memory=False)  # alpha sizes differ
    with pytest.raises(ValueError):
        T.delta_blob(pc, [(256, 500)] + SHAPES[1:], mode, pin_memory=False)
    blob = T.delta_blob(pc, SHAPES, mode, pin_memory=False)
    with pytest.raises(ValueError):
        T.save_delta(tmp_path / "x", blob[:-1], SHAPES, mode)
    with pytest.raises(ValueError):
        T.save_delta(tmp_path / "x", blob, SHAPES, 7)
