"""The allocation-free forward (sq_linear_fwd_static) through the C ABI.

It must give exactly what sq_linear_fwd gives on the same inputs (the same
kernels run, only the scratch lives in the library's static array), on two
calls in a row with the second smaller, including a second call on another
kernel path that reads what the first left in the shared array.
"""
import numpy as np
import pytest
import torch

from synth import gen_activations, gen_payload
from tests.helpers import dev, to_dev_payload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401


def _x(xbits):
    return torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(dev())


@pytest.mark.parametrize("n,k,g,rank,ms", [
    (520, 2048, 32, 32, (300, 5)),      # tile path, then the decode path (M <= 16)
    (256, 1024, 64, 64, (40, 16)),      # streaming small-M path, then decode
    (3072, 3072, 32, 32, (1536, 128)),  # 1536 x 3072 x 3072, then a split-K plan
    (1000, 768, 32, 0, (16, 1)),        # decode twice, rank 0
])
def test_static_forward_equals_workspace_forward(n, k, g, rank, ms):
    import w4_gemm_amd as W
    rng = np.random.default_rng(n + k)
    codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
    if rank == 0:
        upb = dnb = None
    p = to_dev_payload(codes, scales, upb, dnb, g)
    xbits = gen_activations(rng, max(ms), k, 0.01)
    for m in ms:                                  # two calls in a row, the second smaller
        print(f"static forward n{n} k{k} g{g} r{rank} m{m}", flush=True)
        xd = _x(xbits[:m])
        for dt in (torch.float32, torch.bfloat16):
            ref = W.linear_fwd(xd, p, dt)
            got = W.linear_fwd_static(xd, p, dt)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16) if dt == torch.bfloat16 else got,
                               ref.view(torch.int16) if dt == torch.bfloat16 else ref)


def test_static_forward_refuses_oversized_calls():
    import w4_gemm_amd as W
    from w4_gemm_amd import SqError
    rng = np.random.default_rng(3)
    codes, scales, upb, dnb = gen_payload(rng, 6144, 16384, 32, 32)
    p = to_dev_payload(codes, scales, upb, dnb, 32)
    x = torch.zeros((4480, 16384), dtype=torch.bfloat16, device=dev())
    with pytest.raises(SqError):
        W.linear_fwd_static(x, p)
    # the same payload at M = 16 fits and matches
    xb = _x(gen_activations(rng, 16, 16384, 0.005))
    ref = W.linear_fwd(xb, p)
    got = W.linear_fwd_static(xb, p)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
