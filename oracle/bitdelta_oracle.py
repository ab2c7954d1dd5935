"""BitDelta oracle: compression (sign packing + scale) and the fused linear.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, float64
for the floating-point products, Python integers for the exact scale.

Readings of the page taken here:

* Delta is formed in float32: both bf16 operands widen exactly, one IEEE
  float32 subtraction with round-to-nearest-even, subnormals kept.
* sign(0) = +1, also for -0.0; a NaN delta also gets +1 (the test "d < 0"
  is false for it).
* Packing runs along d_in: element c of row r is bit (c mod 64) of 64-bit word
  (c div 64) of row r, least significant bit first; bit value 1 means +1.
  On a little-endian machine this is the same bytes as a uint8/int8 tensor
  [d_out, d_in/8] holding element c at bit (c mod 8) of byte (c div 8).
* The scale is alpha = mean|Delta| over its scope (the whole matrix, or one
  output row).  To make it independent of summation order it is defined
  through the fixed-point magnitudes q = floor(|d| * 2^48), summed exactly,
  then divided by n * 2^48 with one round-to-nearest-even to float32.  This
  differs from the exact mean by less than 2^-48 before the final rounding.
* A scope with a non-finite delta or |d| >= 2^15 gets alpha = NaN with bits
  0x7FC00000.
"""

from __future__ import annotations

import numpy as np

# Bits of the canonical float32 quiet NaN used to mark a scope whose delta is
# non-finite or out of range.
F32_NAN_BITS = 0x7FC00000
# Number of fraction bits of the fixed-point magnitude q = floor(|d| * 2^48).
Q_FRACTION_BITS = 48
# |d| at or above this makes the scope's alpha NaN (keeps each q below 2^63).
ABS_LIMIT = 2.0 ** 15

ALPHA_PER_MATRIX = 0
ALPHA_PER_ROW = 1


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly: bf16 is the top half
    of a float32."""
    b = np.asarray(bits).astype(np.uint16, copy=False)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def delta_f32(w_ft_bits, w_base_bits) -> np.ndarray:
    """Task vector Delta = W_ft - W_base (page: section "Matematiksel temel",
    the Delta equation), as one float32 subtraction per element."""
    a = bf16_bits_to_f32(w_ft_bits)
    b = bf16_bits_to_f32(w_base_bits)
    with np.errstate(invalid="ignore", over="ignore"):
        return (a - b).astype(np.float32, copy=False)


def sign_bits(d: np.ndarray) -> np.ndarray:
    """sign(Delta) as booleans, True meaning +1 (page: section "Matematiksel
    temel", the approximation W_ft ~ W_base + alpha*sign(Delta)).

    sign(0) is +1 (for -0.0 too), and NaN maps to +1: an element is -1 exactly
    when d < 0 holds."""
    with np.errstate(invalid="ignore"):
        return ~(np.asarray(d) < 0)


def pack_sign_bits(bits: np.ndarray) -> np.ndarray:
    """Pack [d_out, d_in] sign booleans into uint64 words [d_out, d_in/64]
    (page: section "Altyapı ayrıntıları", 8 signs per byte along the input
    dimension, so 4096x4096 packs to 4096x512 bytes).

    Element c of a row becomes bit (c mod 64) of word (c div 64)."""
    bits = np.asarray(bits, dtype=bool)
    d_out, d_in = bits.shape
    if d_in % 64 != 0:
        raise ValueError("d_in must be a multiple of 64")
    b = bits.reshape(d_out, d_in // 64, 64).astype(np.uint64)
    place = np.left_shift(np.uint64(1), np.arange(64, dtype=np.uint64))
    # The 64 terms of a word are distinct powers of two, so the sum is exact.
    return (b * place).sum(axis=2, dtype=np.uint64)


def unpack_sign_bits(packed: np.ndarray, d_in: int) -> np.ndarray:
    """Inverse of pack_sign_bits: int8 signs in {+1, -1}, shape [d_out, d_in]."""
    packed = np.asarray(packed, dtype=np.uint64)
    d_out = packed.shape[0]
    if packed.shape[1] * 64 != d_in:
        raise ValueError("packed width does not match d_in")
    shifts = np.arange(64, dtype=np.uint64)
    b = (packed[:, :, None] >> shifts[None, None, :]) & np.uint64(1)
    return np.where(b.reshape(d_out, d_in) == 1, 1, -1).astype(np.int8)


def _bad_mask(d: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return ~np.isfinite(d) | (np.abs(d) >= ABS_LIMIT)


def fixed_point_scope_sums(d: np.ndarray, alpha_mode: int):
    """Exact S = sum of q = floor(|d| * 2^48) over each scope.

    Returns (sums, counts, bad): a list of Python ints (one per scope: each row
    for per-row mode, one for per-matrix mode), the element count n of each
    scope, and a list of booleans marking scopes that hold a non-finite or
    out-of-range delta.

    |d| is a float32, so |d| * 2^48 is exact in float64 and so is its floor;
    the floor stays below 2^63 because |d| < 2^15.  Each q is split into its
    high and low 32-bit halves (both exact in float64), the halves are summed
    in uint64 without overflow, and the two totals are joined as Python ints.
    """
    d = np.asarray(d, dtype=np.float32)
    d_out, d_in = d.shape
    bad_elem = _bad_mask(d)
    mag = np.where(bad_elem, np.float32(0), np.abs(d)).astype(np.float64)
    q = np.floor(mag * 2.0 ** Q_FRACTION_BITS)
    q_hi = np.floor(q / 2.0 ** 32)
    q_lo = q - q_hi * 2.0 ** 32
    hi_rows = q_hi.astype(np.uint64).sum(axis=1, dtype=np.uint64)
    lo_rows = q_lo.astype(np.uint64).sum(axis=1, dtype=np.uint64)
    row_sums = [(int(h) << 32) + int(lo) for h, lo in zip(hi_rows, lo_rows)]
    row_bad = [bool(x) for x in bad_elem.any(axis=1)]
    if alpha_mode == ALPHA_PER_ROW:
        return row_sums, [d_in] * d_out, row_bad
    if alpha_mode == ALPHA_PER_MATRIX:
        return [sum(row_sums)], [d_out * d_in], [any(row_bad)]
    raise ValueError("alpha_mode must be 0 (per matrix) or 1 (per row)")


def rne_ratio_to_f32_bits(s: int, n: int) -> int:
    """float32 bits of s/n rounded to nearest, ties to even; s >= 0, n > 0.

    Long division on integers: find E with 2^E <= s/n < 2^(E+1), take the
    24-bit quotient floor(s/n * 2^(23-E)), and round on the remainder.  Only
    normal results occur for the scales here (s/n >= 2^-76 when s > 0)."""
    if s < 0 or n <= 0:
        raise ValueError("need s >= 0 and n > 0")
    if s == 0:
        return 0
    e = s.bit_length() - n.bit_length()

    def at_least_pow2(exp: int) -> bool:  # s/n >= 2^exp ?
        return s >= (n << exp) if exp >= 0 else (s << -exp) >= n

    if not at_least_pow2(e):
        e -= 1
    shift = 23 - e
    num, den = (s << shift, n) if shift >= 0 else (s, n << -shift)
    q, r = divmod(num, den)
    if 2 * r > den or (2 * r == den and (q & 1)):
        q += 1
    if q == 1 << 24:
        q >>= 1
        e += 1
    if not -126 <= e <= 127:
        raise ValueError("ratio outside the normal float32 range")
    return ((e + 127) << 23) | (q - (1 << 23))


def alpha_from_delta(d: np.ndarray, alpha_mode: int) -> np.ndarray:
    """alpha = (1/n)*||Delta||_1 = mean|Delta| (page: section "Matematiksel
    temel", the alpha equation), one float32 per matrix or per output row
    (page: section "Altyapı ayrıntıları" stores one float32 per output
    dimension; the conceptual kernel in "Sunum mimarisi" accepts either)."""
    sums, counts, bad = fixed_point_scope_sums(d, alpha_mode)
    out = np.empty(len(sums), dtype=np.uint32)
    for i, (s, n, b) in enumerate(zip(sums, counts, bad)):
        out[i] = F32_NAN_BITS if b else rne_ratio_to_f32_bits(s, n << Q_FRACTION_BITS)
    return out.view(np.float32)


def compress(w_ft_bits, w_base_bits, alpha_mode: int):
    """Compression of one weight matrix: returns (packed uint64 [d_out, d_in/64],
    alpha float32 [1] or [d_out])."""
    d = delta_f32(w_ft_bits, w_base_bits)
    return pack_sign_bits(sign_bits(d)), alpha_from_delta(d, alpha_mode)


def _alpha_per_output(alpha, d_out: int, alpha_mode: int) -> np.ndarray:
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1)
    if alpha_mode == ALPHA_PER_MATRIX:
        if a.size != 1:
            raise ValueError("per-matrix alpha must hold one value")
        return np.full(d_out, a[0])
    if alpha_mode == ALPHA_PER_ROW:
        if a.size != d_out:
            raise ValueError("per-row alpha must hold d_out values")
        return a
    raise ValueError("alpha_mode must be 0 or 1")


def linear(x_bits, w_base_bits, packed, alpha, alpha_mode: int) -> np.ndarray:
    """y = x * (W_base + alpha*sign(Delta))^T with no bias (page: section "Sunum
    mimarisi", the conceptual fused kernel), evaluated in float64 in the split
    form  y = x*W_base^T + alpha (.) (x*S^T), S the unpacked signs.

    x: bf16 bits [M, d_in]; w_base: bf16 bits [d_out, d_in]; packed: uint64
    [d_out, d_in/64]; alpha: float32, one value or d_out values.  Any subset of
    output rows may be passed (y[:, o] depends on row o only)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_base_bits).astype(np.float64)
    d_out, d_in = w.shape
    s = unpack_sign_bits(packed, d_in).astype(np.float64)
    a = _alpha_per_output(alpha, d_out, alpha_mode)
    return x @ w.T + (x @ s.T) * a[None, :]


def linear_by_element(x_bits, w_base_bits, packed, alpha, alpha_mode: int) -> np.ndarray:
    """The product straight from its definition, one output at a time:
    y[m, o] = sum_i x[m, i] * W_eff[o, i], where W_eff[o, i] is W_base[o, i]
    plus alpha_o when bit (i mod 64) of word i/64 of row o is set and minus
    alpha_o when it is clear (page: section "Matematiksel temel", the
    approximation of W_ft; section "Altyapı ayrıntıları", the bit layout).
    Reads each sign from its packed word directly and sums in float64.  Slow
    (Python loops over m and o): a cross-check of ``linear`` on tiny shapes."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_base_bits).astype(np.float64)
    words = np.asarray(packed, dtype=np.uint64)
    m_rows, d_in = x.shape
    d_out = w.shape[0]
    a = _alpha_per_output(alpha, d_out, alpha_mode)
    cols = np.arange(d_in)
    y = np.zeros((m_rows, d_out), dtype=np.float64)
    for o in range(d_out):
        bit = (words[o, cols // 64] >> (cols % 64).astype(np.uint64)) & np.uint64(1)
        w_eff = w[o] + np.where(bit == 1, a[o], -a[o])
        for m in range(m_rows):
            y[m, o] = float(np.sum(x[m] * w_eff))
    return y


def f32_to_bf16_bits(f) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values, rounded to the nearest
    bf16 with ties to the even pattern: add 0x7FFF plus the lowest kept bit to
    the float32 bits, then keep the top 16 bits (a carry out of the mantissa
    moves to the next binade, and past the largest finite value to
    infinity).  Every NaN becomes the quiet NaN 0x7FC0."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    return np.where(nan, np.uint64(0x7FC0), rounded).astype(np.uint16)


def reconstruct(w_base_bits, packed, alpha, alpha_mode: int) -> np.ndarray:
    """W_eff = W_base + alpha*sign(Delta), stored as bf16 (page: section
    "Sunum mimarisi": the effective weight of the conceptual fused kernel,
    which a server without the fused kernel writes out before a standard
    matmul; "Matematiksel temel", the approximation W_ft ~ W_base +
    alpha*sign(Delta)).

    Per element: W_base widened to float32 (exact) plus +alpha_o or -alpha_o
    in one float32 addition (nearest, ties to even), then rounded to bf16
    (nearest, ties to even).  Returns bf16 bits, uint16 [d_out, d_in]."""
    w = bf16_bits_to_f32(w_base_bits)
    d_out, d_in = w.shape
    s = unpack_sign_bits(packed, d_in)
    # alpha arrives as float32, so this float64 -> float32 step is exact
    a = _alpha_per_output(alpha, d_out, alpha_mode).astype(np.float32)
    t = np.where(s > 0, a[:, None], -a[:, None]).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        v = (w + t).astype(np.float32, copy=False)
    return f32_to_bf16_bits(v)


def linear_multi(x_bits, variant_ids, w_base_bits, packed_list, alpha_list,
                 alpha_mode: int) -> np.ndarray:
    """Token batch that mixes variants (page: section "Sunum mimarisi", many
    variants' deltas served over one shared base; "Altyapı ayrıntıları",
    per-variant routing).  Token m uses variant v = variant_ids[m]:
    y[m] = x[m]*W_base^T + alpha_v (.) (x[m]*S_v^T); v = -1 means the base model
    alone.  An id outside [-1, V) gives a NaN row."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_base_bits).astype(np.float64)
    d_out, d_in = w.shape
    ids = np.asarray(variant_ids).reshape(-1)
    if ids.size != x.shape[0]:
        raise ValueError("one variant id per token")
    n_var = len(packed_list)
    y = x @ w.T
    signs = {}
    for m, v in enumerate(ids.tolist()):
        if v == -1:
            continue
        if not 0 <= v < n_var:
            y[m, :] = np.nan
            continue
        if v not in signs:
            signs[v] = unpack_sign_bits(packed_list[v], d_in).astype(np.float64)
        a = _alpha_per_output(alpha_list[v], d_out, alpha_mode)
        y[m, :] += (signs[v] @ x[m]) * a
    return y
