"""MonoSoup merge oracle: several fine-tuned checkpoints of one base merged
through rank-r truncations of their task vectors.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy in
float64.

Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
"MonoSoup": for checkpoints W_1 .. W_k of one base, each task vector
Delta_i = W_i - W_base is replaced by its best rank-r approximation tau_i (a
truncated SVD), and the merged weight is W_base + (1/k) * sum_i tau_i.

Readings taken:

* Delta_i is the exact difference of the bf16 values (float64 holds it).
* tau_i is the rank-r truncation of the singular value decomposition (the
  best rank-r approximation in the Frobenius norm); when r is at least the
  rank of Delta_i, tau_i = Delta_i.  It is unique when sigma_r > sigma_{r+1}.
* The merged weight is stored as bf16, rounded to nearest even; the float32
  mean of the truncations is the method's unrounded result.
"""

from __future__ import annotations

import numpy as np

from .bitdelta_oracle import bf16_bits_to_f32, f32_to_bf16_bits


def truncated_svd(d: np.ndarray, rank: int) -> np.ndarray:
    """Best rank-`rank` approximation of a float64 matrix (U_r S_r V_r^T)."""
    if rank <= 0:
        return np.zeros_like(d)
    try:
        u, s, vt = np.linalg.svd(d, full_matrices=False)
    except np.linalg.LinAlgError:
        # LAPACK's divide-and-conquer driver can fail to converge on large
        # matrices; the QR-iteration driver computes the same decomposition
        import scipy.linalg
        u, s, vt = scipy.linalg.svd(d, full_matrices=False, lapack_driver="gesvd")
    r = min(rank, s.size)
    return (u[:, :r] * s[:r]) @ vt[:r]


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values: rounded to float32, then to bf16
    with ties to even.  The two roundings can differ from one direct
    rounding only within 2^-24 relative of a bf16 halfway point; merged
    weights are compared within one bf16 unit for that reason."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def merge(w_fts, w_base, rank: int):
    """(merged bf16 bits [d_out, d_in], mean of the truncations float64) for
    bf16 bit arrays w_fts (a list of k) and w_base."""
    wb = bf16_bits_to_f32(w_base).astype(np.float64)
    taus = [truncated_svd(bf16_bits_to_f32(w).astype(np.float64) - wb, rank) for w in w_fts]
    tau_mean = sum(taus) / len(taus)
    return f64_to_bf16_bits(wb + tau_mean), tau_mean
