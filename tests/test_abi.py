"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call.

Every call below fails argument validation by construction, so no fake
pointer is ever handed to the runtime or a kernel, on any machine.
"""

import ctypes
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import tenant_linear_layers_amd as T

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "bitdelta.h")
A = 0x100000      # 16-byte-aligned addresses that are never dereferenced
B = 0x200000
C = 0x300000
D = 0x400000
E = 0x500000


def test_header_functions_are_exported():
    text = open(HEADER).read()
    names = set(re.findall(r"^\w[\w\s\*]*?\b(bitdelta_\w+)\s*\(", text, flags=re.M))
    assert names == set(T.EXPORTS), names
    L = T.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(11):
        txt = T.status_string(s)
        assert txt and txt != "unknown status"
    assert T.status_string(123) == "unknown status"


def test_workspace_size():
    assert T.compress_workspace_size(4096, 4096, 0) == 4096 * 16
    assert T.compress_workspace_size(4096, 4096, 1) == 0
    assert T.compress_workspace_size(4096, 100, 0) == 0     # invalid shape
    assert T.compress_workspace_size(0, 64, 0) == 0


def test_host_rounding_matches_oracle():
    """The library's rounding routine (the one its kernels use) against the
    oracle's independent long division, on random sums and counts."""
    rng = np.random.default_rng(7)
    for _ in range(4000):
        n = int(rng.integers(1, 1 << 34))
        s = int(rng.integers(0, 1 << 62)) << int(rng.integers(0, 30))
        s += int(rng.integers(0, 1 << 20))
        want = O.rne_ratio_to_f32_bits(s, n << 48) if s else 0
        assert T.ratio_to_f32_bits(s, n) == want, (s, n)
    # exact halfway cases, both parities
    for q in (1 << 23, (1 << 23) + 1, (1 << 24) - 1):
        for n in (1, 3, 4096):
            s = ((2 * q + 1) * n) << 23               # S/(n 2^48) = (q+1/2) 2^-24
            assert T.ratio_to_f32_bits(s, n) == O.rne_ratio_to_f32_bits(s, n << 48)
    assert T.ratio_to_f32_bits(0, 5) == 0
    assert T.ratio_to_f32_bits(5, 0) == 0x7FC00000
    # the mean of |d| for constant |d| = 2^-12 over 4096 elements
    s = 4096 * (1 << 36)
    assert T.ratio_to_f32_bits(s, 4096) == int(np.float32(2.0 ** -12).view(np.uint32))
    assert float(Fraction(s, 4096 << 48)) == 2.0 ** -12


def test_host_rounding_near_float_midpoints():
    """The rounding takes a double-precision quotient unless it lies within a
    few of its last places of a point halfway between two floats, where it
    falls back to long division.  Sums placed exactly on such midpoints and
    then moved by k units of the quotient's last place (k = -20..20, both
    sides of the fallback window) must still round as the oracle's long
    division does; so must random sums over row lengths like d_in."""
    rng = np.random.default_rng(11)
    for _ in range(300):
        n = int(rng.integers(1, 1 << 24))
        m = int(rng.integers(1 << 23, 1 << 24))          # 24-bit significand
        s_mid = (2 * m + 1) * n                            # S/n = m + 1/2
        s_mid <<= int(rng.integers(0, max(1, 63 - s_mid.bit_length())))
        unit = max(1, s_mid >> 52)                         # about one unit of q's last place
        for k in range(-20, 21):
            s = s_mid + k * unit
            if s <= 0:
                continue
            want = O.rne_ratio_to_f32_bits(s, n << 48)
            assert T.ratio_to_f32_bits(s, n) == want, (s, n, k)
    # exact halfway quotients (q = S/n exactly, taken without the long division)
    for n in (64, 4096, 8192, 28672, 3 << 20):
        for _ in range(200):
            m = int(rng.integers(1 << 23, 1 << 24))
            s = ((2 * m + 1) * n) << int(rng.integers(0, 12))
            assert T.ratio_to_f32_bits(s, n) == O.rne_ratio_to_f32_bits(s, n << 48), (s, n)
    for _ in range(6000):
        n = int(rng.choice([64, 192, 4096, 8192, 28672, 1 << 20]))
        s = int(rng.integers(1, 1 << 63))
        assert T.ratio_to_f32_bits(s, n) == O.rne_ratio_to_f32_bits(s, n << 48), (s, n)


def _c(status):
    return int(status)


def test_compress_argument_errors():
    L = T.lib()
    f = L.bitdelta_compress
    assert _c(f(None, B, 4, 64, 1, C, D, None, 0, None)) == 1
    assert _c(f(A, B, 4, 100, 1, C, D, None, 0, None)) == 2      # d_in % 64
    assert _c(f(A, B, 0, 64, 1, C, D, None, 0, None)) == 2       # d_out
    assert _c(f(A, B, 4, 0, 1, C, D, None, 0, None)) == 2
    assert _c(f(A, B, 1 << 31, 64, 1, C, D, None, 0, None)) == 2
    assert _c(f(A, B, 8, (1 << 30) + 64, 1, C, D, None, 0, None)) == 2   # row length cap
    assert _c(f(A, B, 8, 1 << 30, 7, C, D, None, 0, None)) == 4          # passes the shape check
    assert _c(f(A, B, 4, 64, 2, C, D, None, 0, None)) == 4       # mode
    assert _c(f(A + 2, B, 4, 64, 1, C, D, None, 0, None)) == 3   # alignment
    assert _c(f(A, B, 4, 64, 0, C, D, None, 0, None)) == 6       # no workspace
    assert _c(f(A, B, 4, 64, 0, C, D, E, 63, None)) == 6         # too small
    assert _c(f(A, B, 4, 64, 1, A + 64, D, None, 0, None)) == 9  # packed overlaps w_ft


def test_linear_argument_errors():
    f = T.lib().bitdelta_linear
    assert _c(f(A, 4, B, C, D, 1, 8, 64, None, None)) == 1
    assert _c(f(A, 0, B, C, D, 1, 8, 64, E, None)) == 2          # M = 0
    assert _c(f(A, 4, B, C, D, 1, 8, 96, E, None)) == 2          # d_in % 64
    assert _c(f(A, 4, B, C, D, 7, 8, 64, E, None)) == 4
    assert _c(f(A, 4, B, C + 8, D, 1, 8, 64, E, None)) == 3
    assert _c(f(A, 4, B, C, D + 2, 1, 8, 64, E, None)) == 3      # alpha needs 4 bytes
    assert _c(f(A, 4, B, C, D, 1, 8, 64, A, None)) == 9          # y overlaps x
    # The prefill path (M > 64) addresses a 256-row weight tile with 32-bit
    # offsets: d_in above 4194240 is rejected there, but not for M <= 64.
    big = 4194240 + 64
    assert _c(f(A, 65, B, C, D, 1, 8, big, E, None)) == 2
    assert _c(f(A, 65, B, C, D, 7, 8, 4194240, E, None)) == 4    # passes the shape check
    assert _c(f(A, 64, B, C, D, 7, 8, big, E, None)) == 4
    # The decode-shaped path (M <= 64) addresses 16 weight rows and up to 64
    # token rows with 32-bit offsets: d_in above 16777152 is rejected there.
    assert _c(f(A, 1, B, C, D, 1, 8, 16777152 + 64, E, None)) == 2
    assert _c(f(A, 64, B, C, D, 7, 8, 16777152, E, None)) == 4   # passes the shape check


def test_multi_argument_errors():
    f = T.lib().bitdelta_linear_multi
    vp = ctypes.c_void_p
    arr = (vp * 2)(C, C + 4096)
    al = (vp * 2)(D, D + 4096)
    nul = (vp * 2)(C, None)
    pa, aa, na = (ctypes.cast(a, vp) for a in (arr, al, nul))
    assert _c(f(A, 4, B, E, 2, pa, aa, 1, 8, 64, None, None)) == 1
    assert _c(f(A, 4, B, E, 0, pa, aa, 1, 8, 64, E + 65536, None)) == 5
    assert _c(f(A, 4, B, E, 65, pa, aa, 1, 8, 64, E + 65536, None)) == 5
    assert _c(f(A, 4, B, E, 2, na, aa, 1, 8, 64, E + 65536, None)) == 1   # NULL entry
    assert _c(f(A, 4, B + 2, E, 2, pa, aa, 1, 8, 64, E + 65536, None)) == 3
    assert _c(f(A, 4, B, E, 2, pa, aa, 3, 8, 64, E + 65536, None)) == 4
    assert _c(f(A, 4, B, E, 2, pa, aa, 1, 8, 32, E + 65536, None)) == 2
    assert _c(f(A, 4, B, E, 2, pa, aa, 1, 8, 16777152 + 64, E + (1 << 30), None)) == 2
    assert _c(f(A, 4, B, E, 2, pa, aa, 3, 8, 16777152, E + (1 << 30), None)) == 4
    assert _c(f(A, 4, B, E, 2, pa, aa, 1, 8, 64, A, None)) == 9


def test_reconstruct_argument_errors():
    f = T.lib().bitdelta_reconstruct
    assert _c(f(A, C, D, 1, 8, 64, None, None)) == 1
    assert _c(f(None, C, D, 1, 8, 64, E, None)) == 1
    assert _c(f(A, C, D, 1, 8, 96, E, None)) == 2          # d_in % 64
    assert _c(f(A, C, D, 1, 0, 64, E, None)) == 2          # d_out = 0
    assert _c(f(A, C, D, 7, 8, 64, E, None)) == 4
    assert _c(f(A, C + 8, D, 1, 8, 64, E, None)) == 3
    assert _c(f(A, C, D + 2, 1, 8, 64, E, None)) == 3      # alpha needs 4 bytes
    assert _c(f(A, C, D, 1, 8, 64, E + 8, None)) == 3
    assert _c(f(A, C, D, 1, 8, 64, A + 16, None)) == 9     # w_eff overlaps w_base
    assert _c(f(A, C, D, 1, 8, 64, C, None)) == 9          # ... the packed signs
    assert _c(f(A, C, E + 4, 1, 8, 64, E, None)) == 9      # ... per-row alpha


def test_monosoup_argument_checks():
    """bitdelta_monosoup_merge rejects bad arguments before any HIP call
    (the addresses are never dereferenced)."""
    L = T.lib()
    arr = (ctypes.c_void_p * 2)(A, B)
    cast = lambda a: ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    ws = T.monosoup_workspace_size(256, 512, 2, 8)
    assert ws > 0
    assert T.monosoup_workspace_size(256, 512, 2, 33) == 0
    assert T.monosoup_workspace_size(256, 100, 2, 8) == 0

    def call(k=2, rank=8, q=3, d_out=256, d_in=512, omega=C, out=D, tau=None, wsp=E, wsb=ws,
             w=arr):
        return L.bitdelta_monosoup_merge(cast(w), k, ctypes.c_void_p(0x600000), d_out, d_in,
                                         rank, q, ctypes.c_void_p(omega), ctypes.c_void_p(out),
                                         ctypes.c_void_p(tau), ctypes.c_void_p(wsp), wsb, None)
    assert call(rank=0) == 2 and call(rank=33) == 2 and call(k=0) == 2 and call(k=65) == 2
    assert call(q=-1) == 2 and call(q=65) == 2 and call(d_in=100) == 2 and call(d_out=4, rank=8) == 2
    assert call(d_out=65535 * 64 + 1, d_in=64) == 2     # past the merge grid's rows
    assert call(d_out=64, d_in=1 << 24) == 2             # past the product's 32-bit offsets
    assert T.monosoup_workspace_size(64, 1 << 24, 2, 8) == 0
    assert T.monosoup_workspace_size(64, (1 << 24) - 64, 2, 8) > 0
    assert call(omega=0) == 1 and call(out=0) == 1 and call(wsp=0) == 1
    assert call(out=D + 8) == 3 and call(omega=C + 2) == 3
    assert call(wsb=ws - 1) == 6
    assert call(out=B) == 9                               # output over a checkpoint
    nul = (ctypes.c_void_p * 2)(A, None)
    assert call(w=nul) == 1


def test_probe_argument_checks():
    """The calibration probes reject bad arguments before any HIP call."""
    L = T.lib()
    f, g = L.bitdelta_probe_stream_read, L.bitdelta_probe_mfma_bf16
    vp = ctypes.c_void_p
    assert f(vp(0), 1024, 8, vp(B), None) == 1
    assert f(vp(A), 1024, 8, vp(0), None) == 1
    assert f(vp(A), 0, 8, vp(B), None) == 2 and f(vp(A), 1000, 8, vp(B), None) == 2
    assert f(vp(A), 1024, 0, vp(B), None) == 2 and f(vp(A), 1024, (1 << 20) + 1, vp(B), None) == 2
    assert f(vp(A + 8), 1024, 8, vp(B), None) == 3 and f(vp(A), 1024, 8, vp(B + 2), None) == 3
    assert f(vp(A), 4096, 8, vp(A + 512), None) == 9       # sink inside the source
    assert g(8, 16, vp(0), None) == 1
    assert g(0, 16, vp(B), None) == 2 and g(8, 0, vp(B), None) == 2
    assert g(8, (1 << 24) + 1, vp(B), None) == 2 and g(8, 16, vp(B + 1), None) == 3
    h = L.bitdelta_probe_decode_loads
    far = 0x10000000                                        # 32 MiB clear of A..E
    assert h(vp(0), vp(C), vp(D), 0, vp(B), None) == 1
    assert h(vp(far), vp(C), vp(D), 0, vp(0), None) == 1
    assert h(vp(far), vp(C), vp(D), 6, vp(B), None) == 4 and h(vp(far), vp(C), vp(D), -1, vp(B), None) == 4
    assert h(vp(far + 8), vp(C), vp(D), 0, vp(B), None) == 3
    assert h(vp(far), vp(C + 2), vp(D), 0, vp(B), None) == 3
    assert h(vp(far), vp(C), vp(D + 8), 0, vp(B), None) == 3
    assert h(vp(far), vp(C), vp(D), 0, vp(B + 2), None) == 3
    assert h(vp(far), vp(C), vp(D), 0, vp(far + 4096), None) == 9   # sink inside w
    assert h(vp(far), vp(C), vp(D), 0, vp(C + 512), None) == 9      # inside the signs
    assert h(vp(far), vp(C), vp(D), 0, vp(D + 256), None) == 9      # inside x


def test_compress_noalloc_argument_checks():
    """bitdelta_compress_noalloc rejects bad arguments, and per-matrix shapes
    past its 262144-row scratch, before any HIP call."""
    f = T.lib().bitdelta_compress_noalloc
    vp = ctypes.c_void_p
    assert f(vp(0), vp(B), 16, 64, 0, vp(C), vp(D), None) == 1
    assert f(vp(A), vp(B), 16, 100, 0, vp(C), vp(D), None) == 2
    assert f(vp(A), vp(B), 16, 64, 2, vp(C), vp(D), None) == 4
    assert f(vp(A), vp(B), 262145, 64, 0, vp(C), vp(D), None) == 6
    assert f(vp(A + 8), vp(B), 16, 64, 0, vp(C), vp(D), None) == 3
    assert f(vp(A), vp(B), 16, 64, 1, vp(A + 64), vp(D), None) == 9
