"""The alternative kernels kept for A/B measurements, against the oracle:
the vector-ALU GEMV decode (M <= 4) and the operand-layout decode
(BITDELTA_DECODE_KERNEL=valu / operand), and the windowed mixed-batch kernel
(BITDELTA_MULTI_KERNEL=windows).  The switches are read at every call."""

import os

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
import tenant_linear_layers_amd as T
from helpers import assert_y_close, bits16, packed_u64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.lib()


@pytest.fixture
def env():
    saved = {k: os.environ.get(k) for k in ("BITDELTA_DECODE_KERNEL", "BITDELTA_MULTI_KERNEL")}
    yield os.environ
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def _linear_case(shape, m, mode, seed):
    wb, wf = S.small_pair(*shape, 0.02, 1e-3, seed=seed)
    x = S.draw_activations(m, shape[1], S.generator(seed + 1))
    wb, wf, x = (t.to(DEV) for t in (wb, wf, x))
    packed, alpha = T.compress(wf, wb, mode)
    ref = O.linear(bits16(x), bits16(wb), packed_u64(packed), alpha.cpu().numpy(), mode)
    return x, wb, packed, alpha, ref


@pytest.mark.parametrize("kernel,ms", [("valu", [1, 2, 3, 4]), ("operand", [1, 5, 16, 33, 64])])
@pytest.mark.parametrize("shape", [(17, 192), (100, 320), (64, 1024), (1, 64), (4100, 4160)])
def test_decode_alternative_kernels(env, kernel, ms, shape):
    env["BITDELTA_DECODE_KERNEL"] = kernel
    for m in ms:
        mode = (m + shape[0]) % 2
        x, wb, packed, alpha, ref = _linear_case(shape, m, mode, seed=shape[0] + m)
        y = T.linear(x, wb, packed, alpha, mode)
        assert_y_close(y, ref, f"{kernel} decode {shape} M={m}")


@pytest.mark.parametrize("m", [1, 17, 32, 50, 64])
def test_multi_windows_kernel(env, m):
    env["BITDELTA_MULTI_KERNEL"] = "windows"
    g = S.generator(60 + m)
    wb = S.draw_base(130, 512, 0.02, g)
    wfs = [S.draw_finetuned(wb, 2e-4 * (v + 1), g) for v in range(6)]
    wb = wb.to(DEV)
    packs, alphas = zip(*[T.compress(w.to(DEV), wb, 1) for w in wfs])
    ids = np.random.default_rng(m).integers(-1, 6, size=m).astype(np.int32)
    x = S.draw_activations(m, 512, S.generator(61 + m)).to(DEV)
    idt = torch.from_numpy(ids).to(DEV)
    y = T.linear_multi(x, idt, wb, list(packs), list(alphas), 1)
    ref = O.linear_multi(bits16(x), ids, bits16(wb), [packed_u64(p) for p in packs],
                         [a.cpu().numpy() for a in alphas], 1)
    assert_y_close(y, ref, f"windows multi M={m}")


def test_probe_decode_loads_every_mode():
    """The calibration probe of the decode's loads (it computes nothing of the
    method): every load pattern runs on a 4096 x 4096 matrix, twice, and
    leaves the sink alone on ordinary data; a wrong shape is refused by the
    binding before any call."""
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    w = torch.randn(4096, 4096, generator=g, device=DEV).to(torch.bfloat16)
    signs = torch.randint(0, 2 ** 31 - 1, (1 << 19,), generator=g, device=DEV, dtype=torch.int32)
    x = torch.randn(4096, generator=g, device=DEV).to(torch.bfloat16)
    sink = torch.zeros(256, dtype=torch.int32, device=DEV)
    for mode in range(6):
        for _ in range(2):
            T.probe_decode_loads(w, signs, x, mode, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    with pytest.raises(ValueError):
        T.probe_decode_loads(w[:2048], signs, x, 0, sink)
