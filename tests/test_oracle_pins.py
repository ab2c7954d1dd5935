"""Pins of the CPU oracle against what the page and mathematics fix.

Nothing here compares the oracle with itself: each check uses a closed form,
a textbook routine, brute force, a hand-derived fixture under tests/golden/,
or an invariant that a plausible mistake (dropped term, wrong sign, swapped
index, transposed operand, wrong bit order) would break.

Page: "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak" (hanzo.blog).
"""

import os
import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from synthetic import small_pair, bf16_bits, draw_activations, generator

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def bf16_exact(values):
    """bf16 bit patterns of values that bf16 holds exactly."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def f32_rne_of_fraction(fr: Fraction) -> np.float32:
    """Independent rounding of an exact rational to float32 (nearest, ties to
    even) by searching the neighbours of a first guess and comparing exact
    distances.  Different algorithm from the oracle's long division."""
    guess = np.float32(float(fr))
    cands = {guess}
    for _ in range(2):
        for c in list(cands):
            cands.add(np.nextafter(c, np.float32(-np.inf)))
            cands.add(np.nextafter(c, np.float32(np.inf)))
    cands = [c for c in cands if np.isfinite(c)]
    best = min(abs(Fraction(float(c)) - fr) for c in cands)
    ties = [c for c in cands if abs(Fraction(float(c)) - fr) == best]
    if len(ties) == 1:
        return ties[0]
    even = [c for c in ties if (int(f32_bits(c)) & 1) == 0]
    assert len(even) == 1
    return even[0]


def small_case(d_out, d_in, seed, sigma=0.02, b=1e-3):
    w, wft = small_pair(d_out, d_in, sigma, b, seed)
    return bf16_bits(w), bf16_bits(wft)


# ----------------------------------------------------------------- packing
def _pattern_delta(pattern, d_in):
    idx = np.arange(d_in)
    neg = {
        "none": np.zeros(d_in, bool),
        "all": np.ones(d_in, bool),
        "odd": idx % 2 == 1,
        "even": idx % 2 == 0,
        "first": idx == 0,
        "last": idx == d_in - 1,
        "c64": idx == 64,
        "low8": idx < 8,
        "mod8": idx % 8 == 3,
        "zeros": np.zeros(d_in, bool),
    }[pattern]
    base = np.zeros(d_in, np.float32)
    ft = np.where(neg, -1.0, 1.0).astype(np.float32)
    if pattern == "zeros":
        # every delta exactly zero: +0 - +0, and -0 - +0 = -0 on odd elements
        ft = np.where(idx % 2 == 1, np.float32(-0.0), np.float32(0.0))
    return ft, base


def test_pack_hand_derived_words():
    lines = [ln.split("#")[0].split() for ln in open(os.path.join(GOLDEN, "pack_words.txt"))]
    lines = [ln for ln in lines if ln]
    assert len(lines) >= 10
    for ln in lines:
        d_in, pattern, words = int(ln[0]), ln[1], [int(w, 16) for w in ln[2:]]
        ft, base = _pattern_delta(pattern, d_in)
        packed, _ = O.compress(bf16_exact(ft)[None, :], bf16_exact(base)[None, :], 1)
        assert packed.shape == (1, d_in // 64)
        assert [int(w) for w in packed[0]] == words, pattern


def test_negative_zero_and_nan_pack_as_plus():
    d = np.array([[-0.0, 0.0, np.nan, -np.nan, -1e-30, 1e-30] + [1.0] * 58], np.float32)
    bits = O.sign_bits(d)
    assert bits[0, :6].tolist() == [True, True, True, True, False, True]


def test_pack_matches_numpy_packbits():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2, size=(37, 320)).astype(bool)
    packed = O.pack_sign_bits(bits)
    assert sys.byteorder == "little"
    as_bytes = packed.view(np.uint8).reshape(37, 320 // 8)
    ref = np.packbits(bits, axis=1, bitorder="little")
    np.testing.assert_array_equal(as_bytes, ref)


def test_unpack_round_trip_and_popcount():
    wb, wf = small_case(24, 192, seed=5)
    d = O.delta_f32(wf, wb)
    packed, _ = O.compress(wf, wb, 1)
    s = O.unpack_sign_bits(packed, 192)
    np.testing.assert_array_equal(s, np.where(d < 0, -1, 1))
    pop = [sum(bin(int(w)).count("1") for w in row) for row in packed]
    assert pop == (~(d < 0)).sum(axis=1).tolist()


def test_packed_size_is_n_over_8():
    # 4096x4096 packs to 4096x512 bytes (page, section "Altyapı ayrıntıları")
    bits = np.ones((4096, 4096), bool)
    p = O.pack_sign_bits(bits)
    assert p.nbytes == 4096 * 4096 // 8
    assert p.view(np.uint8).reshape(4096, -1).shape == (4096, 512)
    # one bit per weight: 70e9 weights -> 8.75e9 bytes (section "Matematiksel temel")
    assert 70 * 10**9 // 8 == 8_750_000_000
    p2 = O.pack_sign_bits(np.zeros((256, 512), bool))
    assert p2.nbytes == 16384


# ----------------------------------------------------------------- alpha
def test_rounding_hand_derived():
    n_lines = 0
    for ln in open(os.path.join(GOLDEN, "alpha_rounding.txt")):
        f = ln.split("#")[0].split()
        if not f:
            continue
        s, n, want = int(f[0]), int(f[1]), int(f[2], 16)
        assert O.rne_ratio_to_f32_bits(s, n) == want, (s, n)
        n_lines += 1
    assert n_lines >= 10


def test_rounding_matches_search_on_random_ratios():
    rng = np.random.default_rng(3)
    for _ in range(3000):
        n = int(rng.integers(1, 1 << 40)) << int(rng.integers(0, 48))
        s = int(rng.integers(1, 1 << 62)) * int(rng.integers(1, 1 << 20))
        if not 2.0 ** -120 < s / n < 2.0 ** 120:
            continue
        got = O.rne_ratio_to_f32_bits(s, n)
        want = int(f32_bits(f32_rne_of_fraction(Fraction(s, n))))
        assert got == want, (s, n)


@pytest.mark.parametrize("shape,mode", [((3, 64), 1), ((8, 128), 1), ((8, 128), 0), ((5, 256), 0)])
def test_alpha_equals_exact_mean(shape, mode):
    wb, wf = small_case(*shape, seed=shape[0] * 31 + mode)
    d = O.delta_f32(wf, wb)
    # with |d| a multiple of 2^-48 the fixed-point sum is the exact sum
    assert np.all(np.floor(np.abs(d).astype(np.float64) * 2.0 ** 48) == np.abs(d).astype(np.float64) * 2.0 ** 48)
    alpha = O.alpha_from_delta(d, mode)
    rows = [d[r] for r in range(d.shape[0])] if mode == 1 else [d.reshape(-1)]
    for a, r in zip(alpha, rows):
        exact = sum(Fraction(float(abs(v))) for v in r) / len(r)
        assert f32_bits(a) == f32_bits(f32_rne_of_fraction(exact))


def test_alpha_within_half_ulp_of_numpy_mean():
    wb, wf = small_case(512, 4096, seed=2, b=5e-4)
    d = O.delta_f32(wf, wb)
    alpha = O.alpha_from_delta(d, 1).astype(np.float64)
    mean = np.mean(np.abs(d.astype(np.float64)), axis=1)
    ulp = np.spacing(alpha.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(alpha - mean) <= 0.5 * ulp * (1 + 1e-6))
    am = O.alpha_from_delta(d, 0).astype(np.float64)[0]
    mm = np.mean(np.abs(d.astype(np.float64)))
    assert abs(am - mm) <= 0.5 * float(np.spacing(np.float32(am))) * (1 + 1e-6)


def test_alpha_is_least_squares_optimal_scale():
    # argmin_a ||D - a*s||^2 = <D, s>/n; with sign(0)=+1 this is mean|D|.
    wb, wf = small_case(64, 512, seed=9)
    d = O.delta_f32(wf, wb).astype(np.float64)
    packed, alpha = O.compress(wf, wb, 1)
    s = O.unpack_sign_bits(packed, 512).astype(np.float64)
    a_ls = (d * s).sum(axis=1) / 512.0
    a = alpha.astype(np.float64)
    assert np.all(np.abs(a - a_ls) <= np.spacing(alpha).astype(np.float64))

    def loss(scale):
        return ((d - scale[:, None] * s) ** 2).sum(axis=1)

    base = loss(a)
    for f in (1 + 2.0 ** -12, 1 - 2.0 ** -12):
        assert np.all(loss(a * f) >= base - 1e-18)


def test_constant_magnitude_reconstructs_exactly():
    rng = np.random.default_rng(21)
    for m in range(1, 8):
        j = rng.integers(-120, 121, size=(16, 128))
        sgn = rng.choice([-1, 1], size=(16, 128))
        base = (j * 2.0 ** -12).astype(np.float32)
        ft = ((j + sgn * m) * 2.0 ** -12).astype(np.float32)
        wb, wf = bf16_exact(base), bf16_exact(ft)
        for mode in (0, 1):
            packed, alpha = O.compress(wf, wb, mode)
            c = np.float32(m * 2.0 ** -12)
            assert np.all(f32_bits(alpha) == f32_bits(c))
            s = O.unpack_sign_bits(packed, 128).astype(np.float64)
            np.testing.assert_array_equal(s, sgn)
            recon = base.astype(np.float64) + float(c) * s
            np.testing.assert_array_equal(recon, ft.astype(np.float64))


def test_matrix_sum_is_sum_of_row_sums():
    wb, wf = small_case(33, 192, seed=4)
    d = O.delta_f32(wf, wb)
    rows, rn, _ = O.fixed_point_scope_sums(d, 1)
    mat, mn, _ = O.fixed_point_scope_sums(d, 0)
    assert mat == [sum(rows)] and mn == [33 * 192] and rn == [192] * 33
    # brute force: one Python int per element
    brute = sum(int(np.floor(abs(float(v)) * 2.0 ** 48)) for v in d.reshape(-1))
    assert mat[0] == brute


def test_nan_and_out_of_range_scopes():
    wb, wf = small_case(5, 64, seed=1)
    wf = wf.copy()
    wf[1, 5] = 0x7F80                       # +inf in row 1
    wf[2, 7] = bf16_exact([2.0 ** 15])[0]   # |d| >= 2^15 in row 2
    wf[3, 9] = bf16_exact([2.0 ** 14])[0]   # below the limit in row 3
    wf[4, 11] = 0xFFC1                      # a NaN in row 4
    d = O.delta_f32(wf, wb)
    a = f32_bits(O.alpha_from_delta(d, 1))
    assert a[1] == O.F32_NAN_BITS and a[2] == O.F32_NAN_BITS and a[4] == O.F32_NAN_BITS
    assert a[0] != O.F32_NAN_BITS and a[3] != O.F32_NAN_BITS
    assert O.sign_bits(d)[4, 11]            # NaN delta packs as +1
    assert f32_bits(O.alpha_from_delta(d, 0))[0] == O.F32_NAN_BITS


def test_laplace_scale_sanity():
    # E|Delta| = b under the page's Laplace(0, b) model ("Matematiksel temel")
    wb, wf = small_case(256, 4096, seed=2, b=5e-4)
    d = O.delta_f32(wf, wb)
    ratio = float(np.mean(np.abs(d.astype(np.float64)))) / 5e-4
    assert 0.97 < ratio < 1.03


# ----------------------------------------------------------------- linear
def _linear_case(m, d_out, d_in, seed, mode):
    wb, wf = small_case(d_out, d_in, seed=seed)
    x = bf16_bits(draw_activations(m, d_in, generator(seed + 100)))
    packed, alpha = O.compress(wf, wb, mode)
    return x, wb, wf, packed, alpha


@pytest.mark.parametrize("mode", [0, 1])
def test_split_form_equals_sum_by_element(mode):
    x, wb, _, packed, alpha = _linear_case(5, 48, 192, 7, mode)
    y = O.linear(x, wb, packed, alpha, mode)
    yd = O.linear_by_element(x, wb, packed, alpha, mode)
    np.testing.assert_allclose(y, yd, rtol=1e-12, atol=1e-14)


def test_linear_matches_pure_python_triple_loop():
    x, wb, _, packed, alpha = _linear_case(4, 8, 64, 13, 1)
    y = O.linear(x, wb, packed, alpha, 1)
    xf = O.bf16_bits_to_f32(x)
    wf = O.bf16_bits_to_f32(wb)
    for m in range(4):
        for o in range(8):
            acc = 0.0
            for i in range(64):
                bit = (int(packed[o, i // 64]) >> (i % 64)) & 1
                sgn = 1.0 if bit else -1.0
                acc += float(xf[m, i]) * (float(wf[o, i]) + float(alpha[o]) * sgn)
            assert abs(acc - y[m, o]) <= 1e-12 * max(1.0, abs(acc))


def test_alpha_zero_reduces_to_base_product():
    x, wb, _, packed, _ = _linear_case(3, 32, 128, 17, 1)
    y = O.linear(x, wb, packed, np.zeros(32, np.float32), 1)
    ref = O.bf16_bits_to_f32(x).astype(np.float64) @ O.bf16_bits_to_f32(wb).astype(np.float64).T
    np.testing.assert_array_equal(y, ref)


def test_zero_base_small_integer_x_is_exact():
    rng = np.random.default_rng(8)
    d_out, d_in, m = 12, 128, 3
    xi = rng.integers(-8, 9, size=(m, d_in))
    x = bf16_exact(xi.astype(np.float32))
    wb = np.zeros((d_out, d_in), np.uint16)
    sg = rng.choice([-1, 1], size=(d_out, d_in))
    wf = bf16_exact((sg * 0.25).astype(np.float32))
    packed, alpha = O.compress(wf, wb, 0)
    assert float(alpha[0]) == 0.25
    y = O.linear(x, wb, packed, alpha, 0)
    exact = (xi @ sg.T) * 0.25          # integer product, then an exact scaling
    np.testing.assert_array_equal(y, exact.astype(np.float64))


def test_one_hot_rows_extract_weff_columns():
    d_out, d_in = 16, 128
    wb, wf = small_case(d_out, d_in, seed=23)
    packed, alpha = O.compress(wf, wb, 1)
    d = O.delta_f32(wf, wb)
    w = O.bf16_bits_to_f32(wb).astype(np.float64)
    for c in (0, 1, 63, 64, 127):
        x = np.zeros((1, d_in), np.float32)
        x[0, c] = 1.0
        y = O.linear(bf16_exact(x), wb, packed, alpha, 1)[0]
        sgn = np.where(d[:, c] < 0, -1.0, 1.0)   # straight from the delta
        np.testing.assert_array_equal(y, w[:, c] + alpha.astype(np.float64) * sgn)


def test_linear_is_linear_in_x():
    x, wb, _, packed, alpha = _linear_case(2, 24, 128, 29, 0)
    xf = O.bf16_bits_to_f32(x)
    y1 = O.linear(x, wb, packed, alpha, 0)
    x2 = bf16_exact(xf * 2.0)    # doubling is exact in bf16
    y2 = O.linear(x2, wb, packed, alpha, 0)
    np.testing.assert_allclose(y2, 2.0 * y1, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------- multi
def _variants(d_out, d_in, n_var, seed, mode):
    g = generator(seed)
    from synthetic import draw_base, draw_finetuned
    w = draw_base(d_out, d_in, 0.02, g)
    packs, alphas = [], []
    for v in range(n_var):
        wf = draw_finetuned(w, 1e-3 * (1 + v), g)
        p, a = O.compress(bf16_bits(wf), bf16_bits(w), mode)
        packs.append(p)
        alphas.append(a)
    return bf16_bits(w), packs, alphas


@pytest.mark.parametrize("mode", [0, 1])
def test_multi_single_variant_equals_linear(mode):
    wb, packs, alphas = _variants(40, 128, 3, 31, mode)
    x = bf16_bits(draw_activations(6, 128, generator(32)))
    y = O.linear_multi(x, np.full(6, 2, np.int32), wb, packs, alphas, mode)
    np.testing.assert_allclose(y, O.linear(x, wb, packs[2], alphas[2], mode), rtol=1e-12, atol=1e-14)


def test_multi_rows_match_single_token_calls_and_permute():
    wb, packs, alphas = _variants(40, 128, 4, 33, 1)
    x = bf16_bits(draw_activations(7, 128, generator(34)))
    ids = np.array([0, 3, -1, 1, 1, 2, -1], np.int32)
    y = O.linear_multi(x, ids, wb, packs, alphas, 1)
    base = O.bf16_bits_to_f32(x).astype(np.float64) @ O.bf16_bits_to_f32(wb).astype(np.float64).T
    for m, v in enumerate(ids):
        if v < 0:
            np.testing.assert_array_equal(y[m], base[m])
        else:
            ref = O.linear_by_element(x[m:m + 1], wb, packs[v], alphas[v], 1)[0]
            np.testing.assert_allclose(y[m], ref, rtol=1e-12, atol=1e-14)
    perm = np.array([3, 0, 6, 5, 1, 4, 2])
    yp = O.linear_multi(x[perm], ids[perm], wb, packs, alphas, 1)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-13, atol=1e-15)


def test_multi_bad_id_gives_nan_row():
    wb, packs, alphas = _variants(16, 64, 2, 35, 1)
    x = bf16_bits(draw_activations(3, 64, generator(36)))
    y = O.linear_multi(x, np.array([0, 5, -2], np.int32), wb, packs, alphas, 1)
    assert np.all(np.isfinite(y[0])) and np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))


# ------------------------------------------------------- unfused W_eff (bf16)
@pytest.mark.parametrize("f32, bf16", [
    (0x3F800000, 0x3F80),  # 1.0
    (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway, the even neighbour is 1.0
    (0x3F818000, 0x3F82),  # 1 + 3*2^-8: halfway, the even neighbour is above
    (0x3F808001, 0x3F81),  # just above halfway
    (0x3F807FFF, 0x3F80),  # just below halfway
    (0xBF818000, 0xBF82),  # negative ties round the magnitude the same way
    (0x7F7FFFFF, 0x7F80),  # the largest float32 rounds up to +inf
    (0x7F7F7FFF, 0x7F7F),  # below the halfway point of the largest bf16
    (0xFF800000, 0xFF80),  # -inf
    (0x80000000, 0x8000),  # -0
    (0x00000001, 0x0000),  # the smallest subnormal rounds to +0
    (0x00008000, 0x0000),  # subnormal tie, even neighbour 0
    (0x00018000, 0x0002),  # subnormal tie, even neighbour above
    (0x7FC00000, 0x7FC0),  # quiet NaN
    (0xFFC00001, 0x7FC0),  # NaN with sign and payload
    (0x7F800001, 0x7FC0),  # signalling NaN
])
def test_bf16_rounding_hand_derived(f32, bf16):
    f = np.array([f32], dtype=np.uint32).view(np.float32)
    assert int(O.f32_to_bf16_bits(f)[0]) == bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # every exponent, and the patterns on both sides of each halfway point
    u[:4096] = (u[:4096] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[4096:8192] = (u[4096:8192] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.f32_to_bf16_bits(f), ref)


def test_reconstruct_constant_magnitude_gives_w_ft():
    """A delta of constant magnitude c compresses to alpha = c, and W_eff
    rebuilt from it is W_ft itself, bit for bit."""
    rng = np.random.default_rng(23)
    for m in (1, 3, 7):
        j = rng.integers(-120, 121, size=(16, 192))
        sgn = rng.choice([-1, 1], size=(16, 192))
        wb = bf16_exact(j * 2.0 ** -12)
        wf = bf16_exact((j + sgn * m) * 2.0 ** -12)
        for mode in (0, 1):
            packed, alpha = O.compress(wf, wb, mode)
            np.testing.assert_array_equal(O.reconstruct(wb, packed, alpha, mode), wf)


def test_reconstruct_alpha_zero_is_base():
    wb, _ = small_case(24, 128, 3)
    wb = np.where(wb & 0x7FFF == 0, np.uint16(0x3C00), wb)  # no signed zeros
    packed = O.pack_sign_bits(np.random.default_rng(4).random((24, 128)) < 0.5)
    np.testing.assert_array_equal(
        O.reconstruct(wb, packed, np.zeros(24, np.float32), 1), wb)


@pytest.mark.parametrize("mode", [0, 1])
def test_reconstruct_is_a_bf16_neighbour_of_the_exact_sum(mode):
    """Brute force per element: the exact W_base +- alpha (float64 holds it
    exactly here) lies between two adjacent bf16 values; W_eff must be one of
    them, and the nearer one unless the sum lies within float32 rounding
    reach of the halfway point between them."""
    d_out, d_in = 24, 256
    wb, wf = small_case(d_out, d_in, 31)
    packed, alpha = O.compress(wf, wb, mode)
    if mode == 1:  # rows with scales of very different size
        alpha = (alpha * np.float32(2.0) ** np.arange(d_out, dtype=np.float32) % 9).astype(np.float32)
    r = O.reconstruct(wb, packed, alpha, mode)
    w = O.bf16_bits_to_f32(wb).astype(np.float64)
    s = O.unpack_sign_bits(packed, d_in).astype(np.float64)
    a = np.broadcast_to(np.asarray(alpha, np.float64).reshape(-1, 1), (d_out, 1))
    exact = w + s * a
    assert np.all(exact != 0)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    down = np.floor(exact / ulp) * ulp
    up = down + ulp
    got = O.bf16_bits_to_f32(r).astype(np.float64)
    assert np.all((got == down) | (got == up))
    nearer = np.where(exact - down < up - exact, down, up)
    clear = np.abs((exact - down) - ulp / 2) > np.abs(exact) * 2.0 ** -24
    np.testing.assert_array_equal(got[clear], nearer[clear])


def test_reconstruct_rounds_twice_float32_then_bf16():
    """1 + (2^-8 + 2^-30): the float32 sum is exactly halfway between the bf16
    values 1 and 1 + 2^-7 and ties to 1.0, although the exact sum lies above
    the halfway point (a single rounding would give 1 + 2^-7)."""
    wb = bf16_exact(np.full((1, 64), 1.0))
    packed = O.pack_sign_bits(np.ones((1, 64), bool))
    alpha = np.array([2.0 ** -8 + 2.0 ** -30], np.float32)
    assert float(alpha[0]) == 2.0 ** -8 + 2.0 ** -30
    r = O.reconstruct(wb, packed, alpha, 0)
    assert np.all(r == 0x3F80)
    # minus sign: 1 - (2^-8 + 2^-30) rounds in float32 to 1 - 2^-8, which
    # bf16 holds exactly (0x3F7F)
    r = O.reconstruct(wb, O.pack_sign_bits(np.zeros((1, 64), bool)), alpha, 0)
    assert np.all(r == 0x3F7F)


def test_laplace_draw_stays_finite():
    """The Laplace inverse CDF is infinite at u = -1/2, which torch.rand's
    exact zeros would reach (about one draw in 2^24 on the device): the draw
    clamps u to one float32 step inside, so no delta is infinite and the
    largest magnitude is about 16.6 b."""
    import torch
    import synthetic as S
    g = S.generator(123)
    base = torch.zeros(2048, 4096, dtype=torch.bfloat16)
    wf = S.draw_finetuned(base, 1.0, g).float()
    assert torch.isfinite(wf).all()
    assert wf.abs().max().item() <= 16.7
    u = torch.tensor([0.0]) - 0.5                      # the value torch.rand's zero gives
    assert u.clamp(min=S.workloads.U_MIN).item() > -0.5
