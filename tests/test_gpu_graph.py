"""The forward entry points captured in a HIP graph (as the small-M bench
times them): every replay, with the program's own eager work and
synchronizations between replays, must give the eager result bit for bit.
Covers the M <= 16 path (fused and split calls, whose first half is two
device copies), the streaming small-M and tile kernels, and the int8 and
MXFP4 modes."""
import numpy as np
import pytest
import torch

from synth import gen_activations, gen_payload, gen_payload_mx, gen_payload_w8
from tests.helpers import dev, to_dev_payload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def _check_graph(call, out, other):
    """call() writes `out`; other() is unrelated eager work."""
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32)), rep
        other()


@pytest.mark.parametrize("m", [1, 16, 40, 300])
def test_graph_w4_forward(m):
    import w4_gemm_amd as W
    rng = np.random.default_rng(50 + m)
    n, k = 520, 2048
    codes, scales, upb, dnb = gen_payload(rng, n, k, 32, 32)
    p = to_dev_payload(codes, scales, upb, dnb, 32)
    x = _bf16(gen_activations(rng, m, k, 0.01))
    x2 = _bf16(gen_activations(rng, m, k, 0.01))
    ws = torch.empty(W.fwd_workspace_bytes(m, p), dtype=torch.uint8, device=dev())
    ws2 = torch.empty_like(ws)
    for dt in (torch.float32, torch.bfloat16):
        y = torch.empty((m, n), dtype=dt, device=dev())
        y2 = torch.empty_like(y)
        _check_graph(lambda: W.linear_fwd(x, p, out=y, workspace=ws), y,
                     lambda: W.linear_fwd(x2, p, out=y2, workspace=ws2))
    # the split calls in one graph
    y = torch.empty((m, n), dtype=torch.float32, device=dev())
    y2 = torch.empty_like(y)

    def split():
        W.linear_fwd_rotate(x, p, ws)
        W.linear_fwd_contract(m, p, y, ws)
    _check_graph(split, y, lambda: W.linear_fwd(x2, p, out=y2, workspace=ws2))


@pytest.mark.parametrize("m", [1, 300])
def test_graph_w8_and_mx_forward(m):
    import w4_gemm_amd as W
    from w4_gemm_amd import MX4Payload, W8Payload
    rng = np.random.default_rng(60 + m)
    n, k = 300, 1024
    d = dev()
    x = _bf16(gen_activations(rng, m, k, 0.01))
    x2 = _bf16(gen_activations(rng, m, k, 0.01))
    q, s, upb, dnb = gen_payload_w8(rng, n, k, 16)
    p8 = W8Payload(torch.from_numpy(q).to(d), torch.from_numpy(s).to(d), _bf16(upb), _bf16(dnb))
    ws = torch.empty(W.fwd_w8_workspace_bytes(m, p8), dtype=torch.uint8, device=d)
    ws2 = torch.empty_like(ws)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=d)
    y2 = torch.empty_like(y)
    _check_graph(lambda: W.linear_fwd_w8(x, p8, out=y, workspace=ws), y,
                 lambda: W.linear_fwd_w8(x2, p8, out=y2, workspace=ws2))
    c, e, upb, dnb = gen_payload_mx(rng, n, k, 32)
    pm = MX4Payload(torch.from_numpy(c).to(d), torch.from_numpy(e).to(d), _bf16(upb), _bf16(dnb))
    ws = torch.empty(W.fwd_mx4_workspace_bytes(m, pm), dtype=torch.uint8, device=d)
    ws2 = torch.empty_like(ws)
    y = torch.empty((m, n), dtype=torch.float32, device=d)
    y2 = torch.empty_like(y)
    _check_graph(lambda: W.linear_fwd_mx4(x, pm, out=y, workspace=ws), y,
                 lambda: W.linear_fwd_mx4(x2, pm, out=y2, workspace=ws2))
