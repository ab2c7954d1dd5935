"""bitdelta_compress_noalloc (the entry point for callers that cannot
allocate) against bitdelta_compress, through the C ABI: packed signs and
alpha bit for bit, on consecutive calls whose second input is smaller, so a
call never depends on what an earlier call left in the shared scratch."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
import tenant_linear_layers_amd as T
from helpers import alpha_bits, bits16, packed_u64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.lib()


def _pair(d_out, d_in, b, seed):
    wb, wf = S.small_pair(d_out, d_in, 0.02, b, seed)
    return wb.to(DEV), wf.to(DEV)


def _both(wf, wb, mode):
    p_ref, a_ref = T.compress(wf, wb, mode)
    d_out, d_in = wb.shape
    p = torch.full((d_out, d_in // 64), -1, dtype=torch.int64, device=DEV)
    a = torch.full((d_out if mode == 1 else 1,), float("nan"), dtype=torch.float32, device=DEV)
    T.compress_noalloc(wf, wb, mode, p, a)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed_u64(p), packed_u64(p_ref))
    np.testing.assert_array_equal(alpha_bits(a), alpha_bits(a_ref))
    return p, a


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_matches_compress_on_consecutive_calls(mode):
    # a large matrix, then a smaller one: the second call's rows cover only
    # part of what the first left in the scratch
    wb, wf = _pair(3000, 1088, 1e-3, 11)
    _both(wf, wb, mode)
    wb2, wf2 = _pair(200, 512, 4e-4, 12)
    p, a = _both(wf2, wb2, mode)
    # and the small one against the oracle
    p_o, a_o = O.compress(bits16(wf2), bits16(wb2), mode)
    np.testing.assert_array_equal(packed_u64(p), p_o)
    np.testing.assert_array_equal(alpha_bits(a), a_o.view(np.uint32))


def test_noalloc_largest_per_matrix_rows():
    # the scratch's full extent (262144 rows), then a one-row matrix
    wb, wf = _pair(262144, 64, 1e-3, 13)
    _both(wf, wb, 0)
    wb2, wf2 = _pair(1, 64, 1e-3, 14)
    _both(wf2, wb2, 0)


def test_noalloc_rejects_rows_past_scratch():
    wb = torch.zeros(262145, 64, dtype=torch.bfloat16, device=DEV)
    p = torch.empty(262145, 1, dtype=torch.int64, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)
    with pytest.raises(T.BitDeltaError) as e:
        T.compress_noalloc(wb, wb.clone(), 0, p, a)
    assert e.value.status == 6
    # per-row mode uses no scratch and takes the shape
    a2 = torch.empty(262145, dtype=torch.float32, device=DEV)
    T.compress_noalloc(wb, wb.clone(), 1, p, a2)
    torch.cuda.synchronize()
    assert bool((alpha_bits(a2) == 0).all())
