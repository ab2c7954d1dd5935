"""Pins of the MonoSoup merge oracle (CPU): closed forms of the rank-r
truncation and the merge's special cases."""

import numpy as np
import pytest

from oracle import monosoup as M
from oracle.bitdelta_oracle import bf16_bits_to_f32, f32_to_bf16_bits


def test_truncation_of_a_diagonal_keeps_the_largest_magnitudes():
    d = np.diag([2.0, -5.0, 1.0, 3.0])
    np.testing.assert_allclose(M.truncated_svd(d, 2), np.diag([0.0, -5.0, 0.0, 3.0]), atol=1e-12)
    np.testing.assert_allclose(M.truncated_svd(d, 0), np.zeros((4, 4)))
    np.testing.assert_allclose(M.truncated_svd(d, 4), d, atol=1e-12)


def test_truncation_is_exact_on_low_rank_and_permutation_invariant():
    rng = np.random.default_rng(3)
    a, b = rng.normal(size=(40, 3)), rng.normal(size=(30, 3))
    d = a @ b.T
    np.testing.assert_allclose(M.truncated_svd(d, 3), d, atol=1e-10)
    np.testing.assert_allclose(M.truncated_svd(d, 7), d, atol=1e-10)
    full = d + 1e-2 * rng.normal(size=d.shape)
    p = np.eye(40)[rng.permutation(40)] * rng.choice([-1.0, 1.0], 40)
    q = np.eye(30)[rng.permutation(30)]
    np.testing.assert_allclose(M.truncated_svd(p @ full @ q, 3), p @ M.truncated_svd(full, 3) @ q,
                               atol=1e-10)


@pytest.mark.parametrize("r", [1, 4, 9])
def test_truncation_meets_the_eckart_young_residual(r):
    """||D - tau||_F^2 equals the sum of the discarded squared singular
    values, taken here from the eigenvalues of D^T D (another routine), and
    the residual is orthogonal to tau."""
    rng = np.random.default_rng(r)
    d = rng.normal(size=(25, 18))
    t = M.truncated_svd(d, r)
    ev = np.sort(np.linalg.eigvalsh(d.T @ d))[::-1]
    assert abs(np.sum((d - t) ** 2) - ev[r:].sum()) < 1e-9 * ev.sum()
    assert abs(np.sum((d - t) * t)) < 1e-9 * ev.sum()
    assert np.linalg.matrix_rank(t, tol=1e-9) == r


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_merge_special_cases():
    rng = np.random.default_rng(5)
    wb = _bf16(rng.normal(0, 0.02, (24, 16)))
    wf = [_bf16(bf16_bits_to_f32(wb) + rng.normal(0, 1e-3, (24, 16))) for _ in range(3)]
    # full rank, one checkpoint: the checkpoint itself
    m, _ = M.merge(wf[:1], wb, 16)
    np.testing.assert_array_equal(m, wf[0])
    # rank 0: the base
    m, t = M.merge(wf, wb, 0)
    np.testing.assert_array_equal(m, wb)
    assert not t.any()
    # identical checkpoints: one truncation
    m1, t1 = M.merge([wf[1]] * 3, wb, 4)
    m2, t2 = M.merge([wf[1]], wb, 4)
    np.testing.assert_array_equal(m1, m2)
    np.testing.assert_allclose(t1, t2, atol=1e-15)
    # full rank, several checkpoints: the plain average of the deltas
    _, t = M.merge(wf, wb, 16)
    avg = sum(bf16_bits_to_f32(w).astype(np.float64) for w in wf) / 3 - bf16_bits_to_f32(wb)
    np.testing.assert_allclose(t, avg, atol=1e-12)
