"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Packing and alpha are compared bit for bit; outputs within the tolerance in
tests/helpers.py.  Small cases compare every output; the full-size workloads
compare sampled output rows (each output row depends on one weight row only)
and sampled compressed rows (per-row alpha), or stream the whole matrix
through the oracle (per-matrix alpha).
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
import tenant_linear_layers_amd as T
from helpers import alpha_bits, assert_y_close, bits16, packed_u64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.lib()  # fail loudly if the library is missing


def to_dev(*ts):
    return [t.to(DEV) for t in ts]


def check_compress(wf, wb, mode, rows=None):
    """GPU compress vs oracle, bit-exact.  rows: sampled rows (per-row mode)."""
    packed, alpha = T.compress(wf, wb, mode)
    torch.cuda.synchronize()
    if rows is None:
        p_ref, a_ref = O.compress(bits16(wf), bits16(wb), mode)
        np.testing.assert_array_equal(packed_u64(packed), p_ref)
        np.testing.assert_array_equal(alpha_bits(alpha), a_ref.view(np.uint32))
    else:
        assert mode == 1
        ridx = torch.as_tensor(rows, device=DEV)
        p_ref, a_ref = O.compress(bits16(wf[ridx]), bits16(wb[ridx]), 1)
        np.testing.assert_array_equal(packed_u64(packed[ridx]), p_ref)
        np.testing.assert_array_equal(alpha_bits(alpha[ridx]), a_ref.view(np.uint32))
    return packed, alpha


def oracle_y(x, wb, packed, alpha, mode, rows=None):
    if rows is None:
        return O.linear(bits16(x), bits16(wb), packed_u64(packed), alpha.cpu().numpy(), mode)
    ridx = torch.as_tensor(rows, device=DEV)
    a = alpha[ridx] if mode == 1 else alpha
    return O.linear(bits16(x), bits16(wb[ridx]), packed_u64(packed[ridx]), a.cpu().numpy(), mode)


# ---------------------------------------------------------------- workload 1
def test_single_256x512_compress_and_linear():
    wl = S.WORKLOADS["single_256x512"]
    g = S.generator(wl.seed)
    (_, d_out, d_in), = wl.matrices
    wb = S.draw_base(d_out, d_in, wl.sigma, g)
    wf = S.draw_finetuned(wb, wl.b, g)
    x = S.draw_activations(4, d_in, g)
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = check_compress(wf, wb, 0)
    assert packed.numel() * 8 == 16384
    y = T.linear(x, wb, packed, alpha, 0)
    assert_y_close(y, oracle_y(x, wb, packed, alpha, 0), "single_256x512 M=4")


# ---------------------------------------------------------------- workload 2
@pytest.fixture(scope="module")
def proj4096():
    wl = S.WORKLOADS["proj_4096"]
    g = S.generator(wl.seed)
    wb = S.draw_base(4096, 4096, wl.sigma, g)
    wf = S.draw_finetuned(wb, wl.b, g)
    xs = {m: S.draw_activations(m, 4096, g) for m in wl.tokens}
    wb, wf = to_dev(wb, wf)
    return wb, wf, {m: x.to(DEV) for m, x in xs.items()}


def test_proj4096_compress_per_row(proj4096):
    wb, wf, _ = proj4096
    check_compress(wf, wb, 1)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_proj4096_linear(proj4096, m):
    wb, wf, xs = proj4096
    packed, alpha = T.compress(wf, wb, 1)
    y = T.linear(xs[m], wb, packed, alpha, 1)
    assert_y_close(y, oracle_y(xs[m], wb, packed, alpha, 1), f"proj_4096 M={m}")


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("shape", [(1, 64), (3, 128), (17, 192), (33, 576), (5, 1088), (70, 4160),
                                   (71, 2112), (2, 4096), (1, 2048)])
@pytest.mark.parametrize("mode", [0, 1])
def test_compress_ragged_shapes(shape, mode):
    wb, wf = S.small_pair(*shape, 0.02, 1e-3, seed=shape[0] * 7 + shape[1])
    wb, wf = to_dev(wb, wf)
    check_compress(wf, wb, mode)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("d_in", [256, 2048, 4160])
def test_compress_special_values(d_in):
    """Zero deltas of either sign, a constant magnitude, inf, NaN and |d| on
    either side of 2^15; the wider rows are split over two waves."""
    rng = np.random.default_rng(5)
    d_out = 8
    base = rng.normal(0, 0.02, (d_out, d_in)).astype(np.float32)
    wb = _bf16(base)
    # row 0: zero delta (+0 and -0); row 1: constant magnitude 2^-12
    ft = wb.float().cpu().numpy().copy()          # row 0 equal to the base
    j = np.clip(np.round(base[1] * 4096), -200, 200)
    ft[1] = (j + rng.choice([-1, 1], d_in)) / 4096
    wb = wb.clone()
    wb[1] = _bf16(j / 4096)
    wf = _bf16(ft)
    wf[0, ::2] = _bf16(np.zeros(d_in // 2)) * -1.0     # -0 against +/-0 bases
    wb[0, ::2] = 0
    # row 2: +inf, row 3: NaN, row 4: |d| >= 2^15, row 5: |d| just below 2^15
    wf[2, 3] = float("inf")
    wf[3, 9] = float("nan")
    wf[4, 0] = 65536.0
    wb[4, 0] = 0.0
    wf[5, 0] = 16384.0
    wb[5, 0] = -16000.0
    packed, alpha = check_compress(wf, wb, 1)
    a = alpha_bits(alpha)
    assert a[0] == 0 and np.all(packed_u64(packed)[0] == np.uint64(0xFFFFFFFFFFFFFFFF))
    assert alpha.cpu()[1].item() == 2.0 ** -12
    assert a[2] == a[3] == a[4] == 0x7FC00000 and a[5] != 0x7FC00000
    check_compress(wf, wb, 0)


def test_compress_large_deltas_either_side_of_fast_bound():
    """The row sum takes a single 64-bit accumulator while max|d| * d_in <
    2^16 and an exact two-limb recount above; rows on both sides of the
    bound (d_in = 2048: |d| = 20 and |d| = 40) must stay bit-exact."""
    rng = np.random.default_rng(12)
    d_out, d_in = 6, 2048
    base = rng.normal(0, 0.02, (d_out, d_in)).astype(np.float32)
    ft = base + rng.laplace(0, 1e-3, (d_out, d_in)).astype(np.float32)
    ft[1, 5] = base[1, 5] + 20.0
    ft[2, 7] = base[2, 7] - 40.0
    ft[3, :] = base[3, :] + rng.uniform(-31.0, 31.0, d_in).astype(np.float32)
    ft[4, :] = base[4, :] + rng.uniform(-33.0, 33.0, d_in).astype(np.float32)
    wb, wf = _bf16(base), _bf16(ft)
    check_compress(wf, wb, 1)
    check_compress(wf, wb, 0)


def test_compress_is_deterministic():
    wb, wf = S.small_pair(300, 2048, 0.02, 1e-3, seed=77)
    wb, wf = to_dev(wb, wf)
    for mode in (0, 1):
        p1, a1 = T.compress(wf, wb, mode)
        p2, a2 = T.compress(wf, wb, mode)
        assert torch.equal(p1, p2) and torch.equal(a1.view(torch.int32), a2.view(torch.int32))


@pytest.mark.parametrize("shape", [(17, 192), (100, 320), (64, 1024), (1, 64)])
@pytest.mark.parametrize("m", [1, 2, 15, 16, 17, 31, 33, 48, 63, 64])
def test_linear_decode_ragged(shape, m):
    mode = (shape[0] + m) % 2
    wb, wf = S.small_pair(*shape, 0.02, 1e-3, seed=shape[0] + m)
    x = S.draw_activations(m, shape[1], S.generator(m))
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = T.compress(wf, wb, mode)
    y = T.linear(x, wb, packed, alpha, mode)
    assert_y_close(y, oracle_y(x, wb, packed, alpha, mode), f"decode {shape} M={m}")


@pytest.mark.parametrize("shape", [(1000, 512), (4100, 256), (33, 8192), (48, 8256), (20, 64)])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_linear_decode_interleaved_rows(shape, m):
    """Up to 16 tokens with d_in <= 8192 a workgroup takes four chunks of 4
    rows spread over the matrix (chunks past d_out partly or wholly empty)
    and starts each wave at a rotated block; 8256 takes contiguous rows.
    Every output is compared, starting from a NaN-filled y."""
    d_out, d_in = shape
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=d_out + m)
    x = S.draw_activations(m, d_in, S.generator(7 * m))
    wb, wf, x = to_dev(wb, wf, x)
    for mode in (0, 1):
        packed, alpha = T.compress(wf, wb, mode)
        y = torch.full((m, d_out), float("nan"), dtype=torch.bfloat16, device=DEV)
        T.linear(x, wb, packed, alpha, mode, y=y)
        assert_y_close(y, oracle_y(x, wb, packed, alpha, mode), f"decode {shape} M={m} mode {mode}")


@pytest.mark.parametrize("shape", [(4100, 4032), (5120, 64), (4096, 1088), (4096, 4096)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_linear_decode_four_wave_rows(shape, m):
    """Up to 4 tokens on 256..320 groups of 16 rows (four-wave workgroups):
    ragged and 64-wide final blocks, a single block of d_in, and every token
    count up to 4.  Every output is compared, starting from a NaN-filled y."""
    d_out, d_in = shape
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=d_in + m)
    x = S.draw_activations(m, d_in, S.generator(11 * m))
    wb, wf, x = to_dev(wb, wf, x)
    for mode in (0, 1):
        packed, alpha = T.compress(wf, wb, mode)
        y = torch.full((m, d_out), float("nan"), dtype=torch.bfloat16, device=DEV)
        T.linear(x, wb, packed, alpha, mode, y=y)
        assert_y_close(y, oracle_y(x, wb, packed, alpha, mode), f"decode {shape} M={m} mode {mode}")


@pytest.mark.parametrize("m", [1, 16, 64])
def test_linear_decode_longest_rows(m):
    """d_in = 16777152, the longest row the decode-shaped path (up to 64
    tokens) accepts: its 32-bit x offsets come within 8 KB of 2^31 at 64
    tokens (x is 2 GiB), and the weight rows take the contiguous-row form.
    The first, a middle and the last row against the oracle."""
    d_out, d_in = 17, 16777152
    mode = m % 2
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=60 + m, device=DEV)
    packed, alpha = T.compress(wf, wb, mode)
    del wf
    x = S.draw_activations(m, d_in, S.generator(61 + m, DEV), DEV)
    y = T.linear(x, wb, packed, alpha, mode)
    rows = [0, 9, 16]
    assert_y_close(y[:, rows], oracle_y(x, wb, packed, alpha, mode, rows=rows),
                   f"decode d_in={d_in} M={m}")


def test_linear_prefill_longest_rows():
    """d_in = 4194240, the longest row the prefill path (more than 64
    tokens) accepts: a 256-row weight tile and a 256-token x tile then span
    2^31 - 32 KB with 32-bit offsets.  300 rows (a full 256-row tile and a
    ragged one), 65 tokens; sampled rows of both tiles against the oracle."""
    d_out, d_in, m = 300, 4194240, 65
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=62, device=DEV)
    packed, alpha = T.compress(wf, wb, 0)
    del wf
    x = S.draw_activations(m, d_in, S.generator(63, DEV), DEV)
    y = T.linear(x, wb, packed, alpha, 0)
    rows = [0, 255, 256, 299]
    assert_y_close(y[:, rows], oracle_y(x, wb, packed, alpha, 0, rows=rows),
                   f"prefill d_in={d_in} M={m}")


@pytest.mark.parametrize("shape", [(130, 192), (257, 640), (128, 64)])
@pytest.mark.parametrize("m", [65, 100, 256, 300, 513])
def test_linear_prefill_ragged(shape, m):
    mode = (shape[0] + m) % 2
    wb, wf = S.small_pair(*shape, 0.02, 1e-3, seed=shape[1] + m)
    x = S.draw_activations(m, shape[1], S.generator(m + 1))
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = T.compress(wf, wb, mode)
    y = T.linear(x, wb, packed, alpha, mode)
    assert_y_close(y, oracle_y(x, wb, packed, alpha, mode), f"prefill {shape} M={m}")


# Prefill shapes that take each tile path of the launcher: 512 x 128
# producer/consumer tiles over whole rounds of the 256 CUs with the remaining
# rows on 256-token tiles, producer/consumer tiles alone, 256 x 256 tiles over
# whole rounds with the rest as 256 x 128 producer/consumer tiles (token
# padding rules out the 512-row tiles at M = 600), 256 x 128 producer/consumer
# tiles alone (4096 x 4096, M = 2048; and M = 200 with 193 row tiles, the last
# one ragged, over an odd number of 64-wide steps) and 256 x 64 tiles
# (2048 x 2048, M = 2048: 128-wide tiles would fill half a round).
# (M, d_out, d_in, mode, first row past the first launch or None)
PREFILL_PATHS = [
    (1000, 16677, 192, 1, 16384),
    (1024, 16384, 320, 0, None),
    (272, 33024, 192, 0, 32768),
    (600, 22056, 128, 1, 21760),
    (2048, 4096, 4096, 1, None),
    (200, 24600, 192, 1, None),
    (2048, 2048, 320, 0, None),
]


@pytest.mark.parametrize("case", PREFILL_PATHS, ids=lambda c: f"M{c[0]}_{c[1]}x{c[2]}")
def test_linear_prefill_tile_paths(case):
    m, d_out, d_in, mode, split = case
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=d_out + m)
    x = S.draw_activations(m, d_in, S.generator(m + 5))
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = T.compress(wf, wb, mode)
    y = T.linear(x, wb, packed, alpha, mode)
    rows = set(_sample_rows(d_out, 40, d_in + m).tolist()) | {127, 128, 255, 256}
    if split is not None:
        rows |= {split - 129, split - 128, split - 1, split, split + 1, split + 127, split + 128}
    rows = np.array(sorted(r for r in rows if 0 <= r < d_out))
    assert_y_close(y[:, torch.as_tensor(rows, device=DEV)],
                   oracle_y(x, wb, packed, alpha, mode, rows=rows), f"prefill path {case}")


# Products whose producer/consumer tiles are dealt to the 8 XCDs in blocks
# of g token-tile groups times 8/g weight-tile groups (the launcher picks g
# by what the L2s fetch): g = 4 and g = 8 on 256 x 128 tiles, g = 2 on
# 512 x 128 tiles.  A tile dealt twice or never would leave part of y
# unwritten (y is allocated empty), so every output is compared.
# (M, d_out, d_in, mode)
PREFILL_XCD_BLOCKS = [
    (4096, 2048, 256, 0),
    (8192, 1024, 256, 1),
    (4096, 4096, 192, 0),
]


@pytest.mark.parametrize("case", PREFILL_XCD_BLOCKS, ids=lambda c: f"M{c[0]}_{c[1]}x{c[2]}")
def test_linear_prefill_xcd_blocks_full_output(case):
    m, d_out, d_in, mode = case
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=d_out + m + 3)
    x = S.draw_activations(m, d_in, S.generator(m + 9))
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = T.compress(wf, wb, mode)
    y = torch.full((m, d_out), float("nan"), dtype=torch.bfloat16, device=DEV)
    T.linear(x, wb, packed, alpha, mode, y=y)
    assert_y_close(y, oracle_y(x, wb, packed, alpha, mode), f"prefill XCD blocks {case}")


def test_linear_prefill_tall_x_few_rows():
    """M = 200000 tokens over 128 rows: the whole rounds of producer/consumer
    tiles hold fewer tiles than one weight tile's column of token tiles, so
    the launcher takes 256-token tiles for the whole product (a zero-row
    producer/consumer launch before the guard).  Every output is compared."""
    m, d_out, d_in = 200000, 128, 64
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=77)
    x = S.draw_activations(m, d_in, S.generator(78))
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = T.compress(wf, wb, 0)
    y = torch.full((m, d_out), float("nan"), dtype=torch.bfloat16, device=DEV)
    T.linear(x, wb, packed, alpha, 0, y=y)
    assert_y_close(y, oracle_y(x, wb, packed, alpha, 0), "prefill tall x, few rows")


def test_linear_prefill_large_x_prefetch():
    """x of more than 64 MiB (1024 x 32832) takes the producer/consumer tiles
    with x prefetched into L2 two steps ahead; 513 steps (odd)."""
    m, d_out, d_in = 1024, 16384, 32832
    g = S.generator(71, DEV)
    wb = S.draw_base(d_out, d_in, 0.02, g, DEV)
    wf = S.draw_finetuned(wb, 1e-3, g)
    x = S.draw_activations(m, d_in, g, DEV)
    packed, alpha = T.compress(wf, wb, 1)
    del wf
    y = T.linear(x, wb, packed, alpha, 1)
    rows = np.array(sorted(set(_sample_rows(d_out, 24, 72).tolist()) | {127, 128, 8191, 8192}))
    assert_y_close(y[:, torch.as_tensor(rows, device=DEV)],
                   oracle_y(x, wb, packed, alpha, 1, rows=rows), "prefill large x")


@pytest.mark.parametrize("m", [3, 300])
def test_linear_one_hot_extracts_columns(m):
    """x = e_c picks column c of W_eff: any bit-order, axis or layout slip in
    either kernel shows up here."""
    d_out, d_in = 48, 256
    wb, wf = S.small_pair(d_out, d_in, 0.02, 1e-3, seed=91)
    cols = [(7 * i + 3) % d_in for i in range(m)]
    x = np.zeros((m, d_in), np.float32)
    x[np.arange(m), cols] = 1.0
    wb, wf = to_dev(wb, wf)
    xd = _bf16(x)
    packed, alpha = T.compress(wf, wb, 1)
    y = T.linear(xd, wb, packed, alpha, 1).float().cpu().numpy()
    d = O.delta_f32(bits16(wf), bits16(wb))
    w = O.bf16_bits_to_f32(bits16(wb)).astype(np.float64)
    a = alpha.cpu().numpy().astype(np.float64)
    for i, c in enumerate(cols):
        ref = w[:, c] + a * np.where(d[:, c] < 0, -1.0, 1.0)
        assert np.allclose(y[i], ref, rtol=2 ** -8, atol=1e-7), (i, c)


# ---------------------------------------------------------------- multi
def _variants(d_out, d_in, n_var, seed, mode):
    g = S.generator(seed)
    wb = S.draw_base(d_out, d_in, 0.02, g)
    wfs = [S.draw_finetuned(wb, 2e-4 * (v + 1), g) for v in range(n_var)]
    wb = wb.to(DEV)
    packs, alphas = [], []
    for wf in wfs:
        p, a = T.compress(wf.to(DEV), wb, mode)
        packs.append(p)
        alphas.append(a)
    return wb, packs, alphas


def _multi_ref(x, ids, wb, packs, alphas, mode):
    return O.linear_multi(bits16(x), ids.cpu().numpy(), bits16(wb),
                          [packed_u64(p) for p in packs], [a.cpu().numpy() for a in alphas], mode)


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 50, 64, 100, 130])
@pytest.mark.parametrize("shape", [(40, 192), (130, 512)])
def test_multi_mixed_ids(m, shape):
    mode = m % 2
    wb, packs, alphas = _variants(*shape, 5, seed=m + shape[0], mode=mode)
    rng = np.random.default_rng(m)
    ids = rng.integers(-1, 5, size=m).astype(np.int32)
    if m > 3:
        ids[2] = 7           # invalid id -> NaN row
        ids[3] = -5
    x = S.draw_activations(m, shape[1], S.generator(m + 2)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = T.linear_multi(x, idt, wb, packs, alphas, mode)
    assert_y_close(y, _multi_ref(x, idt, wb, packs, alphas, mode), f"multi {shape} M={m}")


def test_multi_single_variant_matches_linear():
    """A batch of one variant through the mixed kernel does the same
    arithmetic as the single-variant kernel; only the grouping of the float32
    partial sums differs, so outputs agree to one bf16 step."""
    wb, packs, alphas = _variants(96, 384, 3, seed=5, mode=1)
    x = S.draw_activations(40, 384, S.generator(6)).to(DEV)
    ids = torch.full((40,), 1, dtype=torch.int32, device=DEV)
    y_multi = T.linear_multi(x, ids, wb, packs, alphas, 1).float()
    y_single = T.linear(x, wb, packs[1], alphas[1], 1).float()
    step = torch.abs(y_single) * 2.0 ** -7 + 1e-30
    assert torch.all(torch.abs(y_multi - y_single) <= step)
    assert (y_multi != y_single).float().mean().item() < 0.05


def test_multi_zipf_mix_many_variants():
    wb, packs, alphas = _variants(200, 1024, 14, seed=9, mode=1)
    ids = torch.from_numpy(S.zipf_ids(64, 14, seed=10)).to(DEV)
    x = S.draw_activations(64, 1024, S.generator(11)).to(DEV)
    y = T.linear_multi(x, ids, wb, packs, alphas, 1)
    assert_y_close(y, _multi_ref(x, ids, wb, packs, alphas, 1), "multi zipf 14 variants")


@pytest.mark.parametrize("m", [5, 33, 64])
def test_multi_wide_ragged(m):
    """d_out >= 8192 takes the two-row-tile workgroups: ragged last workgroup
    (8200 rows), a final half block of d_in (192 = 128 + 64), several token
    tiles, base-only and invalid ids."""
    mode = m % 2
    wb, packs, alphas = _variants(8200, 192, 6, seed=70 + m, mode=mode)
    rng = np.random.default_rng(70 + m)
    ids = rng.integers(-1, 6, size=m).astype(np.int32)
    ids[1] = 9
    x = S.draw_activations(m, 192, S.generator(71 + m)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = T.linear_multi(x, idt, wb, packs, alphas, mode)
    assert_y_close(y, _multi_ref(x, idt, wb, packs, alphas, mode), f"multi wide M={m}")


@pytest.mark.parametrize("shape", [(200, 1024), (8192, 320)])
def test_multi_more_distinct_variants_than_prefetched(shape):
    """40 variants, 40 of them present in a 64-token batch: more distinct
    variants than the kernel prefetches per block (the rest load on demand)."""
    wb, packs, alphas = _variants(*shape, 40, seed=80, mode=1)
    ids = np.concatenate([np.arange(40), np.arange(24)]).astype(np.int32)
    np.random.default_rng(81).shuffle(ids)
    x = S.draw_activations(64, shape[1], S.generator(82)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = T.linear_multi(x, idt, wb, packs, alphas, 1)
    assert_y_close(y, _multi_ref(x, idt, wb, packs, alphas, 1), f"multi 40 variants {shape}")


@pytest.mark.parametrize("shape", [(12345, 192), (24600, 128)])
@pytest.mark.parametrize("m", [20, 32, 50, 64])
def test_multi_many_row_groups_full_output(shape, m):
    """More 16-row groups than the GPU holds at once (772 and 1538, the last
    one ragged), with a base-only token: y starts as NaN and every output is
    compared.  From 33 tokens these take the four-wave workgroups."""
    mode = m % 2
    wb, packs, alphas = _variants(*shape, 9, seed=95 + m, mode=mode)
    ids = S.zipf_ids(m, 9, seed=96 + m)
    ids[0] = -1
    x = S.draw_activations(m, shape[1], S.generator(97 + m)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = torch.full((m, shape[0]), float("nan"), dtype=torch.bfloat16, device=DEV)
    T.linear_multi(x, idt, wb, packs, alphas, mode, y=y)
    assert_y_close(y, _multi_ref(x, idt, wb, packs, alphas, mode), f"multi rounds {shape} M={m}")


@pytest.mark.parametrize("shape", [(300, 320), (5200, 192)])
@pytest.mark.parametrize("m", [16, 32, 64])
def test_multi_every_token_its_own_variant_of_64(shape, m):
    """The largest variant table (64 entries): every token on a variant of
    its own, so each 16-token tile holds 16 pairs and the pairs take several
    batches; 325 row groups take the four-wave workgroups, 19 the eight-wave
    ones, and 192 ends in a 64-wide block.  Every output is compared,
    starting from a NaN-filled y."""
    mode = m % 2
    wb, packs, alphas = _variants(*shape, 64, seed=40 + m, mode=mode)
    ids = np.random.default_rng(41 + m).permutation(64)[:m].astype(np.int32)
    x = S.draw_activations(m, shape[1], S.generator(42 + m)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = torch.full((m, shape[0]), float("nan"), dtype=torch.bfloat16, device=DEV)
    T.linear_multi(x, idt, wb, packs, alphas, mode, y=y)
    assert_y_close(y, _multi_ref(x, idt, wb, packs, alphas, mode), f"multi 64 variants {shape} M={m}")


def test_multi_longest_rows():
    """A mixed batch at d_in = 16777152, the longest row bitdelta_linear_multi
    accepts: 64 tokens over 3 variants and base-only tokens, x of 2 GiB.
    The first, a middle and the last row against the oracle."""
    d_out, d_in, m = 17, 16777152, 64
    g = S.generator(64, DEV)
    wb = S.draw_base(d_out, d_in, 0.02, g, DEV)
    packs, alphas = [], []
    for v in range(3):
        wf = S.draw_finetuned(wb, 2e-4 * (v + 1), g)
        p, a = T.compress(wf, wb, 1)
        del wf
        packs.append(p)
        alphas.append(a)
    ids = np.random.default_rng(65).integers(-1, 3, size=m).astype(np.int32)
    x = S.draw_activations(m, d_in, S.generator(66, DEV), DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = T.linear_multi(x, idt, wb, packs, alphas, 1)
    rows = torch.as_tensor([0, 9, 16], device=DEV)
    ref = O.linear_multi(bits16(x), ids, bits16(wb[rows]), [packed_u64(p[rows]) for p in packs],
                         [a[rows].cpu().numpy() for a in alphas], 1)
    assert_y_close(y[:, rows], ref, f"multi d_in={d_in} M={m}")


def _pattern_ids(kind, m):
    """Variant-id patterns that exercise how a batch is cut into (16-token
    tile, variant) pairs."""
    rng = np.random.default_rng(len(kind) + m)
    if kind == "long_run":       # one variant's run spans several tiles
        ids = np.concatenate([np.full(40, 3), np.full(10, 0), np.full(6, -1),
                              np.arange(4, 12)])[:m]
    elif kind == "base_tile":    # a whole tile of base-only tokens between variants
        ids = np.concatenate([np.full(8, 1), np.full(16, -1), np.arange(2, 10), np.full(16, 5),
                              np.arange(6, 22)])[:m]
    elif kind == "all_base":
        ids = np.full(m, -1)
    elif kind == "all_invalid":
        ids = np.full(m, 99)
    elif kind == "distinct":     # every token its own variant (one pair per token)
        ids = np.arange(m) % 20
    else:
        raise ValueError(kind)
    ids = ids.astype(np.int32)
    rng.shuffle(ids)
    return ids


@pytest.mark.parametrize("kind", ["long_run", "base_tile", "all_base", "all_invalid", "distinct"])
@pytest.mark.parametrize("m", [48, 64])
def test_multi_pair_patterns(kind, m):
    mode = m % 2
    wb, packs, alphas = _variants(300, 320, 20, seed=90 + m, mode=mode)
    ids = _pattern_ids(kind, m)
    x = S.draw_activations(m, 320, S.generator(91 + m)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = T.linear_multi(x, idt, wb, packs, alphas, mode)
    ref = _multi_ref(x, idt, wb, packs, alphas, mode)
    if kind == "all_invalid":
        assert bool(torch.isnan(y.float()).all())
        return
    assert_y_close(y, ref, f"multi pairs {kind} M={m}")


# ---------------------------------------------------------------- workloads 3, 4
def _sample_rows(d_out, k, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(d_out, size=min(k, d_out), replace=False)
    rows[:2] = [0, d_out - 1]
    return np.sort(rows)


def test_layer70b_multi_full_size():
    """14 variants of one 70B-shaped layer, M=32 Zipf(1.1) mix: every one of
    the 70 compressions checked bit-exact on sampled rows, every linear on
    sampled output rows."""
    wl = S.WORKLOADS["layer70b_multi"]
    g = S.generator(wl.seed, DEV)
    bases = S.draw_layer_bases(wl, g, DEV)
    scales = S.variant_scales(wl)
    packs = [[None] * len(bases) for _ in scales]
    alphas = [[None] * len(bases) for _ in scales]
    for v, i, wf in S.iter_finetuned(bases, scales, g):
        rows = _sample_rows(wf.shape[0], 6, 1000 * v + i)
        packs[v][i], alphas[v][i] = check_compress(wf, bases[i], 1, rows=rows)
        del wf
    xs = S.draw_layer_inputs(wl, 32, g, DEV)
    ids = torch.from_numpy(S.zipf_ids(32, wl.n_variants, wl.seed)).to(DEV)
    ids_np = ids.cpu().numpy()
    for i, (name, d_out, d_in) in enumerate(wl.matrices):
        y = T.linear_multi(xs[i], ids, bases[i], [packs[v][i] for v in range(len(scales))],
                           [alphas[v][i] for v in range(len(scales))], 1)
        rows = _sample_rows(d_out, 48, 7 + i)
        ridx = torch.as_tensor(rows, device=DEV)
        ref = O.linear_multi(bits16(xs[i]), ids_np, bits16(bases[i][ridx]),
                             [packed_u64(packs[v][i][ridx]) for v in range(len(scales))],
                             [alphas[v][i][ridx].cpu().numpy() for v in range(len(scales))], 1)
        assert_y_close(y[:, ridx], ref, f"layer70b_multi {name}")


def test_layer70b_decode_full_size():
    """One variant of a 70B-shaped layer (per-row alpha) through the decode
    kernels at M = 1, 4, 16, as the layer decode benchmark runs it, and at
    M = 32 and 64 (the pairs kernel with every token on variant 0): every
    compression bit-exact on sampled rows, every output on sampled rows."""
    wl = S.WORKLOADS["layer70b_decode"]
    g = S.generator(wl.seed, DEV)
    bases = S.draw_layer_bases(wl, g, DEV)
    packs, alphas = [], []
    for _, i, wf in S.iter_finetuned(bases, S.variant_scales(wl), g):
        rows = _sample_rows(wf.shape[0], 6, 500 + i)
        p, a = check_compress(wf, bases[i], 1, rows=rows)
        packs.append(p)
        alphas.append(a)
        del wf
    xs = S.draw_layer_inputs(wl, 64, g, DEV)
    for i, (name, d_out, d_in) in enumerate(wl.matrices):
        rows = _sample_rows(d_out, 48, 600 + i)
        for m in tuple(wl.tokens) + (32, 64):
            y = T.linear(xs[i][:m], bases[i], packs[i], alphas[i], 1)
            ref = oracle_y(xs[i][:m], bases[i], packs[i], alphas[i], 1, rows=rows)
            assert_y_close(y[:, torch.as_tensor(rows, device=DEV)], ref,
                           f"layer70b_decode {name} M={m}")


@pytest.mark.parametrize("shape", [(10240, 8192), (8192, 8192)])
def test_decode_small_m_back_to_back_full_output(shape):
    """Few-token decode (M = 1, 3, 6, 8: the kernels that keep two blocks of
    W_base and x in flight per wave) of four variants of one base, launched
    back to back with x hot in the cache, as a per-variant grouping of a
    mixed batch runs them.  Every output is compared with the oracle (row
    chunks of the float64 product).  A refill of a stage whose last reads
    were still in flight once corrupted a few outputs in each such run."""
    d_out, d_in = shape
    g = S.generator(d_out + 3, DEV)
    wb = S.draw_base(d_out, d_in, 0.015, g, DEV)
    variants = []
    for b in (2e-4, 5e-4, 1e-3, 2e-3):
        wf = S.draw_finetuned(wb, b, g)
        variants.append(T.compress(wf, wb, 1))
        del wf
    x = S.draw_activations(8, d_in, g, DEV)
    for m in (1, 3, 6, 8):
        ys = [T.linear(x[:m], wb, p, a, 1) for p, a in variants]
        torch.cuda.synchronize()
        for v, ((p, a), y) in enumerate(zip(variants, ys)):
            for r0 in range(0, d_out, 2048):
                rows = np.arange(r0, min(r0 + 2048, d_out))
                ref = oracle_y(x[:m], wb, p, a, 1, rows=rows)
                assert_y_close(y[:, r0:r0 + len(rows)], ref,
                               f"{d_out}x{d_in} M={m} variant {v} rows {r0}..")


def _progress(msg):
    import sys
    sys.__stderr__.write(f"  [stack70b] {msg}\n")
    sys.__stderr__.flush()


def test_stack70b_multi_full_size():
    """The whole 80-layer 70B-shaped stack resident on the GPU (137 GB of
    W_base and 14 packed variants of 8.56 GB each), M = 64 tokens with a
    Zipf(1.1) variant mix per layer: every one of the 5600 compressions
    checked bit-exact on sampled rows (per-row alpha), every one of the 400
    mixed-variant linears on sampled output rows."""
    wl = S.WORKLOADS["stack70b_multi"]
    need = 262 * 10**9
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    g = S.generator(wl.seed, DEV)
    stack = S.draw_stack_bases(wl, g, DEV)
    scales = S.variant_scales(wl)
    nv, nm = len(scales), len(wl.matrices)
    packs = [[[None] * nm for _ in range(nv)] for _ in range(wl.layers)]
    alphas = [[[None] * nm for _ in range(nv)] for _ in range(wl.layers)]
    try:
        for l, v, i, wf in S.iter_stack_finetuned(stack, scales, g):
            rows = _sample_rows(wf.shape[0], 3, 100000 * l + 100 * v + i)
            packs[l][v][i], alphas[l][v][i] = check_compress(wf, stack[l][i], 1, rows=rows)
            del wf
            if v == nv - 1 and i == nm - 1 and l % 10 == 9:
                _progress(f"layers 0..{l} drawn and compressed")
        xs = S.draw_stack_inputs(wl, 64, g, DEV)
        ids = torch.from_numpy(S.zipf_ids(64, nv, wl.seed)).to(DEV)
        ids_np = ids.cpu().numpy()
        for l in range(wl.layers):
            for i, (name, d_out, d_in) in enumerate(wl.matrices):
                y = T.linear_multi(xs[l][i], ids, stack[l][i], [packs[l][v][i] for v in range(nv)],
                                   [alphas[l][v][i] for v in range(nv)], 1)
                rows = _sample_rows(d_out, 8, 31 * l + i)
                ridx = torch.as_tensor(rows, device=DEV)
                ref = O.linear_multi(bits16(xs[l][i]), ids_np, bits16(stack[l][i][ridx]),
                                     [packed_u64(packs[l][v][i][ridx]) for v in range(nv)],
                                     [alphas[l][v][i][ridx].cpu().numpy() for v in range(nv)], 1)
                assert_y_close(y[:, ridx], ref, f"stack70b_multi layer {l} {name}")
            if l % 20 == 19:
                _progress(f"linears of layers 0..{l} checked")
    finally:
        del stack, packs, alphas
        torch.cuda.empty_cache()


def _oracle_alpha_streamed(wf, wb, chunk=2048):
    """Per-matrix alpha through the oracle, rows streamed in chunks: the
    matrix sum is the sum of the row sums."""
    total, bad = 0, False
    for r0 in range(0, wf.shape[0], chunk):
        d = O.delta_f32(bits16(wf[r0:r0 + chunk]), bits16(wb[r0:r0 + chunk]))
        sums, _, flags = O.fixed_point_scope_sums(d, 1)
        total += sum(sums)
        bad = bad or any(flags)
    n = wf.shape[0] * wf.shape[1]
    return O.F32_NAN_BITS if bad else O.rne_ratio_to_f32_bits(total, n << O.Q_FRACTION_BITS)


def test_layer70b_prefill_full_size():
    """One variant of one 70B-shaped layer, per-matrix alpha, M=2048 through
    the prefill GEMM: alpha bit-exact over each whole matrix, packing on
    sampled rows, outputs on sampled rows."""
    wl = S.WORKLOADS["layer70b_prefill"]
    g = S.generator(wl.seed, DEV)
    bases = S.draw_layer_bases(wl, g, DEV)
    packs, alphas = [None] * 5, [None] * 5
    for v, i, wf in S.iter_finetuned(bases, S.variant_scales(wl), g):
        packs[i], alphas[i] = T.compress(wf, bases[i], 0)
        assert alpha_bits(alphas[i])[0] == _oracle_alpha_streamed(wf, bases[i])
        rows = _sample_rows(wf.shape[0], 6, 3 + i)
        ridx = torch.as_tensor(rows, device=DEV)
        p_ref, _ = O.compress(bits16(wf[ridx]), bits16(bases[i][ridx]), 1)
        np.testing.assert_array_equal(packed_u64(packs[i][ridx]), p_ref)
        del wf
    xs = S.draw_layer_inputs(wl, 2048, g, DEV)
    for i, (name, d_out, d_in) in enumerate(wl.matrices):
        y = T.linear(xs[i], bases[i], packs[i], alphas[i], 0)
        rows = _sample_rows(d_out, 32, 11 + i)
        assert_y_close(y[:, torch.as_tensor(rows, device=DEV)],
                       oracle_y(xs[i], bases[i], packs[i], alphas[i], 0, rows=rows),
                       f"layer70b_prefill {name}")


# ---------------------------------------------------------------- unfused W_eff
def check_reconstruct(wb, packed, alpha, mode, rows=None):
    """GPU W_eff vs oracle, bit for bit (NaN positions compared as NaN).
    rows: sampled rows (W_eff row o depends on row o only)."""
    w_eff = T.reconstruct(wb, packed, alpha, mode)
    torch.cuda.synchronize()
    if rows is None:
        ref = O.reconstruct(bits16(wb), packed_u64(packed), alpha.cpu().numpy(), mode)
        got = bits16(w_eff)
    else:
        ridx = torch.as_tensor(rows, device=DEV)
        a = alpha[ridx] if mode == 1 else alpha
        ref = O.reconstruct(bits16(wb[ridx]), packed_u64(packed[ridx]), a.cpu().numpy(), mode)
        got = bits16(w_eff[ridx])
    nan_ref = (ref & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal((got & 0x7FFF) > 0x7F80, nan_ref)
    np.testing.assert_array_equal(got[~nan_ref], ref[~nan_ref])
    return w_eff


# 8-weight pieces per row: 8 .. 2048, one or two workgroups per row, 1, 2 or 4
# pieces per thread, last workgroup of a row partly past it
@pytest.mark.parametrize("shape", [(1, 64), (17, 192), (100, 320), (3, 2112), (5, 4096),
                                   (7, 8256), (2, 16384)])
@pytest.mark.parametrize("mode", [0, 1])
def test_reconstruct_ragged(shape, mode):
    wb, wf = S.small_pair(*shape, 0.02, 1e-3, seed=shape[0] * 13 + shape[1] + mode)
    wb, wf = to_dev(wb, wf)
    packed, alpha = T.compress(wf, wb, mode)
    check_reconstruct(wb, packed, alpha, mode)


def test_reconstruct_constant_magnitude_gives_w_ft():
    """A delta of constant magnitude compresses to alpha = |delta| and W_eff
    rebuilt on the GPU is W_ft, bit for bit (no oracle involved)."""
    rng = np.random.default_rng(17)
    j = rng.integers(-120, 121, size=(40, 1024))
    sgn = rng.choice([-1, 1], size=(40, 1024))
    wb = _bf16(j * 2.0 ** -12)
    wf = _bf16((j + 5 * sgn) * 2.0 ** -12)
    for mode in (0, 1):
        packed, alpha = T.compress(wf, wb, mode)
        assert torch.equal(T.reconstruct(wb, packed, alpha, mode).view(torch.int16),
                           wf.view(torch.int16))


@pytest.mark.parametrize("mode", [0, 1])
def test_reconstruct_nan_alpha_scope(mode):
    wb, wf = S.small_pair(12, 576, 0.02, 1e-3, seed=9)
    wf[5, 100] = float("inf")
    wb, wf = to_dev(wb, wf)
    packed, alpha = T.compress(wf, wb, mode)
    w_eff = check_reconstruct(wb, packed, alpha, mode)
    nan_rows = torch.isnan(w_eff.float()).all(dim=1).cpu().numpy()
    expect = np.ones(12, bool) if mode == 0 else np.arange(12) == 5
    np.testing.assert_array_equal(nan_rows, expect)


def test_reconstruct_is_what_prefill_multiplies():
    """x times the materialised W_eff (float64 on the host) agrees with the
    fused prefill GEMM, which rebuilds the same bf16 W_eff tiles in LDS."""
    wb, wf = S.small_pair(300, 640, 0.02, 1e-3, seed=19)
    x = S.draw_activations(300, 640, S.generator(20))
    wb, wf, x = to_dev(wb, wf, x)
    packed, alpha = T.compress(wf, wb, 1)
    w_eff = T.reconstruct(wb, packed, alpha, 1)
    y = T.linear(x, wb, packed, alpha, 1)
    ref = (O.bf16_bits_to_f32(bits16(x)).astype(np.float64)
           @ O.bf16_bits_to_f32(bits16(w_eff)).astype(np.float64).T)
    rel, mx = assert_y_close(y, ref, "prefill vs materialised W_eff")
    assert rel < 2e-3  # only y's bf16 rounding and float32 accumulation differ


def test_proj4096_reconstruct(proj4096):
    wb, wf, _ = proj4096
    packed, alpha = T.compress(wf, wb, 1)
    check_reconstruct(wb, packed, alpha, 1, rows=_sample_rows(4096, 64, 5))


def test_reconstruct_gate_full_size():
    """28672 x 8192 (the 70B-shaped gate projection), per-matrix alpha:
    sampled rows bit for bit."""
    g = S.generator(61, DEV)
    wb = S.draw_base(28672, 8192, 0.015, g, DEV)
    wf = S.draw_finetuned(wb, 1e-3, g)
    packed, alpha = T.compress(wf, wb, 0)
    del wf
    check_reconstruct(wb, packed, alpha, 0, rows=_sample_rows(28672, 24, 62))


def test_binding_rejects_wrong_sizes():
    """The C ABI sees pointers only; the binding checks every tensor's size
    before any launch, so a short output or operand is an error, not an
    out-of-bounds access."""
    wb, wf = to_dev(*S.small_pair(32, 128, 0.02, 1e-3, seed=3))
    x = S.draw_activations(4, 128, S.generator(4)).to(DEV)
    packed, alpha = T.compress(wf, wb, 1)
    short_y = torch.empty(4, 31, dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(4, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        T.linear(x, wb, packed, alpha, 1, y=short_y)
    with pytest.raises(ValueError):
        T.linear(x, wb, packed[:31], alpha, 1)
    with pytest.raises(ValueError):
        T.linear(x, wb, packed, alpha[:31], 1)
    with pytest.raises(ValueError):
        T.linear(x, wb, packed, alpha, 0)             # per-matrix mode needs one alpha
    with pytest.raises(ValueError):
        T.linear_multi(x, ids, wb, [packed], [alpha[:1]], 1)
    with pytest.raises(ValueError):
        T.linear_multi(x, ids, wb, [packed], [alpha], 1, y=short_y)
    with pytest.raises(ValueError):
        T.reconstruct(wb, packed, alpha, 1, w_eff=torch.empty(32, 64, dtype=torch.bfloat16,
                                                               device=DEV))
    with pytest.raises(ValueError):
        T.compress(wf, wb, 1, packed=torch.empty(32, 1, dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):
        T.compress(wf, wb, 0, alpha=torch.empty(32, dtype=torch.float32, device=DEV))


# ---------------------------------------------------------------- graph capture
def test_graph_replays_match_eager():
    """Every entry point captured in one HIP graph: each replay, with eager
    work and synchronisations in between, equals the eager results bit for
    bit (the kernels use no memset and no host-side state)."""
    wb, packs, alphas = _variants(96, 512, 3, seed=41, mode=0)
    wf = S.draw_finetuned(wb.cpu(), 1e-3, S.generator(42)).to(DEV)
    x4 = S.draw_activations(4, 512, S.generator(43)).to(DEV)
    x100 = S.draw_activations(100, 512, S.generator(44)).to(DEV)
    ids = torch.tensor([0, 2, -1, 1], dtype=torch.int32, device=DEV)
    outs = dict(p=torch.empty_like(packs[0]), a=torch.empty_like(alphas[0]),
                y4=torch.empty(4, 96, dtype=torch.bfloat16, device=DEV),
                y100=torch.empty(100, 96, dtype=torch.bfloat16, device=DEV),
                ym=torch.empty(4, 96, dtype=torch.bfloat16, device=DEV),
                we=torch.empty(96, 512, dtype=torch.bfloat16, device=DEV))
    ws = torch.empty(T.compress_workspace_size(96, 512, 0), dtype=torch.uint8, device=DEV)

    def run():
        T.compress(wf, wb, 0, packed=outs["p"], alpha=outs["a"], workspace=ws)
        T.linear(x4, wb, packs[1], alphas[1], 0, y=outs["y4"])
        T.linear(x100, wb, packs[2], alphas[2], 0, y=outs["y100"])
        T.linear_multi(x4, ids, wb, packs, alphas, 0, y=outs["ym"])
        T.reconstruct(wb, packs[0], alphas[0], 0, w_eff=outs["we"])

    run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for v in outs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
        _ = (x100.float() @ x100.float().T).sum().item()   # eager work between replays
