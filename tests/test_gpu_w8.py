"""Device parity of the int8-residual mode (SquareQ README, "v3.1 -
int8-residual mode") through the C ABI against the CPU oracle.

Bars, as for the W4 mode:
  * quantize: codes, fp16 row scales and fraction indices bit-exact on every
    tie-certified row (codes within a half-integer tie may take either
    neighbour); uncertified rows must be admissible;
  * reconstruct: bf16 W_hat within 1e-3 relative Frobenius of the oracle's
    exact W_hat rounded to bf16, at most 1 bf16 ulp per element;
  * forward: fp32 y within 2e-3 relative Frobenius (cos >= 0.9999) of the
    exact fp64 y and within 1e-5 of the oracle on the same fp16 operands;
    bf16 y equal to round-to-nearest-even of the fp32 y.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen_activations, gen_payload_w8, gen_weight, f32_to_bf16_bits
from tests.helpers import bf16_tensor_to_f64, dev, ulp_bf16

pytestmark = pytest.mark.gpu

Y_TOL, COS_TOL, DIAG_TOL, WHAT_TOL = 2e-3, 0.9999, 1e-5, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401  (fails loudly if libsq.so is missing)


def _bf16_dev(bits):
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def _payload(q, scales, upb, dnb):
    from w4_gemm_amd import W8Payload
    d = dev()
    return W8Payload(torch.from_numpy(np.ascontiguousarray(q, dtype=np.int8)).to(d),
                     torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float16)).to(d),
                     _bf16_dev(upb), _bf16_dev(dnb))


def _fp64(q, scales, upb, dnb, k):
    up = O.bf16_decode(upb) if upb is not None else np.zeros((q.shape[0], 0))
    dn = O.bf16_decode(dnb) if dnb is not None else np.zeros((k, 0))
    return q.astype(np.float64), O.fp16_decode(np.asarray(scales)), up, dn


def _factors(rng, n, k, rank):
    if rank == 0:
        return None, None, np.zeros((n, 0)), np.zeros((k, 0))
    upb = f32_to_bf16_bits((rng.standard_normal((n, rank)) * 0.3).astype(np.float32))
    dnb = f32_to_bf16_bits((rng.standard_normal((k, rank)) * 0.3).astype(np.float32))
    return upb, dnb, O.bf16_decode(upb), O.bf16_decode(dnb)


# ------------------------------------------------------------------ quantizer
def _check_quant(w, upb, dnb, up, dn, tag, rows=None):
    import w4_gemm_amd as W
    d = dev()
    p, fidx, flags = W.quantize_weight_w8(torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(d),
                                          _bf16_dev(upb), _bf16_dev(dnb))
    torch.cuda.synchronize()
    assert int(flags[0]) == 0
    rows = np.arange(w.shape[0]) if rows is None else rows
    r = O.residual(w[rows], up[rows], dn)
    res = O.quantize_residual_w8(r)
    ri = torch.from_numpy(rows).to(d)
    rep = O.check_device_quant_w8(r, res, p.codes[ri].cpu().numpy(),
                                  p.scales[ri].cpu().numpy().astype(np.float64), fidx[ri].cpu().numpy())
    print(tag, rep)
    assert rep["ok"], rep
    return p


def test_w8_quantize_shapes_and_ranks():
    rng = np.random.default_rng(21)
    for (n, k, rank) in [(100, 768, 16), (33, 256, 0), (64, 2048, 32), (200, 512, 64), (1, 1280, 16)]:
        w = gen_weight(rng, n, k, 4)
        if n < rank:
            # a single row has no rank-16 split: arbitrary bf16 factors instead
            upb, dnb, up, dn = _factors(rng, n, k, rank)
        elif rank:
            up, dn = O.svd_init(w, rank)
            from tests.helpers import bf16_bits_of
            upb, dnb = bf16_bits_of(up), bf16_bits_of(dn)
        else:
            upb = dnb = None
            up, dn = np.zeros((n, 0)), np.zeros((k, 0))
        _check_quant(w, upb, dnb, up, dn, f"n{n} k{k} r{rank}")


def test_w8_quantize_edge_rows():
    # an all-zero row (scale 0, codes 0), a row on the int8 grid of a
    # candidate scale, a row with one dominant value, a negative-heavy row
    rng = np.random.default_rng(22)
    n, k = 16, 512
    r = rng.standard_normal((n, k)) * 0.05
    r[0] = 0.0
    s = np.float64(np.float16(100.0 / 12700))
    r[1] = np.clip(np.rint(rng.standard_normal(k) * 40), -127, 127) * s
    r[1, 3] = 127 * s
    r[2, 5] = 30.0
    r[3] = -np.abs(r[3])
    w = O.rotate(r).astype(np.float32).astype(np.float64)   # H is its own inverse
    _check_quant(w, None, None, np.zeros((n, 0)), np.zeros((k, 0)), "edge rows")


def test_w8_quantize_flags():
    import w4_gemm_amd as W
    d = dev()
    w = torch.zeros((16, 256), dtype=torch.float32, device=d)
    w[2, 7] = float("nan")
    _, _, flags = W.quantize_weight_w8(w, None, None)
    torch.cuda.synchronize()
    assert int(flags[0]) & 1
    w = torch.zeros((16, 256), dtype=torch.float32, device=d)
    w[5, :] = 1e7                      # rotated DC 1.6e8 -> absmax/127 > 65504
    _, _, flags = W.quantize_weight_w8(w, None, None)
    torch.cuda.synchronize()
    assert int(flags[0]) & 2


# ------------------------------------------------------------------ reconstruct
def _check_reconstruct(q, scales, upb, dnb, tag, rows=None):
    import w4_gemm_amd as W
    n, k = q.shape
    what = W.reconstruct_bf16_w8(_payload(q, scales, upb, dnb))
    torch.cuda.synchronize()
    rows = np.arange(n) if rows is None else rows
    got = bf16_tensor_to_f64(what[torch.from_numpy(rows).to(dev())])
    qf, s, up, dn = _fp64(q[rows], np.asarray(scales)[rows], None if upb is None else upb[rows], dnb, k)
    exact = O.reconstruct_w8(qf, s, up, dn)
    ref = O.bf16_round(exact)
    e = O.rel_fro(got, ref)
    print(f"{tag}: reconstruct relF vs bf16(oracle) = {e:.3e}")
    assert e <= WHAT_TOL
    assert np.all(np.abs(got - ref) <= ulp_bf16(ref))
    assert O.cosine(got, exact) > 0.99999


def test_w8_reconstruct_shapes_and_ranks():
    rng = np.random.default_rng(23)
    for (n, k, rank) in [(100, 768, 16), (33, 256, 0), (64, 2048, 32), (200, 512, 64), (17, 1024, 16)]:
        q, scales, upb, dnb = gen_payload_w8(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        _check_reconstruct(q, scales, upb, dnb, f"n{n} k{k} r{rank}")


def test_w8_reconstruct_extreme_codes():
    # every code at -128 or 127: the butterfly sums reach 2^15 in magnitude
    rng = np.random.default_rng(24)
    n, k = 32, 512
    q = np.where(rng.random((n, k)) < 0.5, -128, 127).astype(np.int8)
    q[0] = -128
    q[1] = 127
    scales = np.full(n, 1e-3, np.float16)
    _check_reconstruct(q, scales, None, None, "extreme codes")


# ------------------------------------------------------------------ forward
def _fwd_checks(xbits, q, scales, upb, dnb, rows=None, tag=""):
    import w4_gemm_amd as W
    k = q.shape[1]
    p = _payload(q, scales, upb, dnb)
    xd = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(dev())
    y32 = W.linear_fwd_w8(xd, p, torch.float32)
    y16 = W.linear_fwd_w8(xd, p, torch.bfloat16)
    torch.cuda.synchronize()
    y32h = y32.cpu().numpy().astype(np.float64)
    y16h = bf16_tensor_to_f64(y16)
    assert np.all(np.isfinite(y32h))
    assert np.array_equal(y16h, O.bf16_round(y32h))
    rows = np.arange(xbits.shape[0]) if rows is None else rows
    x = O.bf16_decode(xbits[rows])
    qf, s, up, dn = _fp64(q, scales, upb, dnb, k)
    ref = O.forward_w8(x, qf, s, up, dn)
    diag = O.forward_w8_fp16_operands(x, qf, s, up, dn)
    got = y32h[rows]
    e, cs, ed = O.rel_fro(got, ref), O.cosine(got, ref), O.rel_fro(got, diag)
    print(f"{tag}: relF={e:.3e} cos={cs:.7f} vs-fp16-operands={ed:.3e}")
    assert e <= Y_TOL and cs >= COS_TOL and ed <= DIAG_TOL
    return y32h


def test_w8_fwd_decode_shapes():
    # M <= 16: the decode kernel on the int8 payload; N ragged against its
    # 256-row workgroups and 64-row waves, K slices with a short last slice,
    # every rank
    rng = np.random.default_rng(28)
    for (n, k, rank) in [(1, 256, 16), (200, 3328, 32), (520, 1024, 64), (256, 2304, 0),
                         (300, 4096, 16)]:
        q, scales, upb, dnb = gen_payload_w8(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, 16, k, 0.01)
        for m in (1, 2, 5, 16):
            _fwd_checks(xbits[:m], q, scales, upb, dnb, tag=f"decode m{m} n{n} k{k} r{rank}")


def test_w8_fwd_small_m():
    # M <= 64: the decode kernel (M <= 16), then the streaming contraction
    # with two and four 16-row tiles
    rng = np.random.default_rng(25)
    for (n, k, rank) in [(200, 1280, 16), (64, 2048, 32), (300, 768, 0), (33, 256, 64)]:
        q, scales, upb, dnb = gen_payload_w8(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, 128, k, 0.01)
        for m in (1, 5, 17, 33, 64, 65, 128):
            _fwd_checks(xbits[:m], q, scales, upb, dnb, tag=f"m{m} n{n} k{k} r{rank}")


def test_w8_fwd_tiles_and_splits():
    # M > 64: the 256-column tile kernel, with and without split K, ragged M and N
    rng = np.random.default_rng(26)
    for (m, n, k, rank) in [(65, 256, 2048, 16), (300, 520, 1024, 16), (600, 1100, 512, 32),
                            (130, 33, 768, 0), (257, 300, 4096, 64)]:
        q, scales, upb, dnb = gen_payload_w8(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, m, k, 0.01)
        _fwd_checks(xbits, q, scales, upb, dnb, tag=f"m{m} n{n} k{k} r{rank}")



def test_w8_fwd_mid_m_plans():
    # mid-size M with long K (224- and 256-row tiles, with and without split-K)
    rng = np.random.default_rng(27)
    for (m, n, k, rank) in [(1500, 1540, 4096, 16), (2000, 1800, 6144, 32), (2000, 4100, 1024, 0)]:
        q, scales, upb, dnb = gen_payload_w8(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, m, k, 0.01)
        rows = np.sort(rng.choice(m, 24, replace=False))
        _fwd_checks(xbits, q, scales, upb, dnb, rows=rows, tag=f"m{m} n{n} k{k} r{rank}")


def test_w8_end_to_end_quantized_layer():
    # device quantizer -> device forward and reconstruct of its own payload
    import w4_gemm_amd as W
    rng = np.random.default_rng(27)
    n, k, m, rank = 192, 1024, 96, 16
    w = gen_weight(rng, n, k, 4)
    up, dn = O.svd_init(w, rank)
    from tests.helpers import bf16_bits_of
    upb, dnb = bf16_bits_of(up), bf16_bits_of(dn)
    p = _check_quant(w, upb, dnb, up, dn, "e2e")
    q = p.codes.cpu().numpy()
    scales = p.scales.cpu().numpy()
    xbits = gen_activations(rng, m, k, 0.01)
    y = _fwd_checks(xbits, q, scales, upb, dnb, tag="e2e fwd")
    _check_reconstruct(q, scales, upb, dnb, "e2e reconstruct")
    # and the layer approximates the original weight: y close to x @ W^T
    x = O.bf16_decode(xbits)
    yw = x @ w.astype(np.float64).T
    assert O.rel_fro(y, yw) < 2e-2


def test_w8_full_size_sampled():
    # the MLP-up shape 4480 x 16384 x 6144 with rank 16: whole layer on the
    # GPU, the oracle on sampled rows
    import w4_gemm_amd as W
    rng = np.random.default_rng(28)
    m, n, k, rank = 4480, 16384, 6144, 16
    q, scales, upb, dnb = gen_payload_w8(rng, n, k, rank)
    xbits = gen_activations(rng, m, k, 0.005)
    p = _payload(q, scales, upb, dnb)
    xd = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(dev())
    y = W.linear_fwd_w8(xd, p, torch.float32)
    what = W.reconstruct_bf16_w8(p)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(m, 24, replace=False))
    x = O.bf16_decode(xbits[rows])
    qf, s, up, dn = _fp64(q, scales, upb, dnb, k)
    got = y[torch.from_numpy(rows).to(dev())].cpu().numpy().astype(np.float64)
    ref = O.forward_w8(x, qf, s, up, dn)
    e, cs = O.rel_fro(got, ref), O.cosine(got, ref)
    print(f"full-size fwd sampled: relF={e:.3e} cos={cs:.7f}")
    assert e <= Y_TOL and cs >= COS_TOL
    wr = np.sort(rng.choice(n, 64, replace=False))
    gw = bf16_tensor_to_f64(what[torch.from_numpy(wr).to(dev())])
    exact = O.reconstruct_w8(qf[wr], s[wr], up[wr], dn)
    ref = O.bf16_round(exact)
    assert O.rel_fro(gw, ref) <= WHAT_TOL
    assert np.all(np.abs(gw - ref) <= ulp_bf16(ref))
