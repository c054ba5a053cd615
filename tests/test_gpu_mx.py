"""Device parity of the MXFP4 mode (SquareQ README, "SquareQ v3 - W4", the
FP4 alternative of the "Residual codecs" bullet, as OCP MXFP4) through the C
ABI against the CPU oracle.

Bars:
  * quantizers (weights and rotated activations): E8M0 exponents and E2M1
    nibbles bit-exact on every certified block; a value within 1e-5 of a
    rounding midpoint may take either neighbour; a block whose absmax is
    within 1e-5 of a power of two may take the adjacent exponent with
    codes consistent with it;
  * reconstruct: bf16 W_hat within 1e-3 relative Frobenius of the oracle's
    exact W_hat rounded to bf16, at most 1 bf16 ulp per element;
  * forward: fp32 y within 1e-5 (relative, per row) of the oracle's exact
    FP4 product on rows whose rotated activations hold no near-midpoint
    value and no block absmax near a power of two; on the other rows every
    element within the deviation that the admissible choices at those
    values allow (one grid step, at most 2 block scales, per near value;
    a doubled scale for a whole uncertain block) plus fp32 accumulation
    error; bf16 y equal to RNE of the fp32 y.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import f32_to_bf16_bits, gen_activations, gen_payload_mx, gen_weight
from tests.helpers import bf16_bits_of, bf16_tensor_to_f64, dev, ulp_bf16

pytestmark = pytest.mark.gpu

WHAT_TOL, ROW_TOL, ACC_TOL = 1e-3, 1e-5, 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401  (fails loudly if libsq.so is missing)


def _bf16_dev(bits):
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def _payload(codes, exps, upb, dnb):
    from w4_gemm_amd import MX4Payload
    d = dev()
    return MX4Payload(torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).to(d),
                      torch.from_numpy(np.ascontiguousarray(exps, np.uint8)).to(d),
                      _bf16_dev(upb), _bf16_dev(dnb))


def _factors(rng, n, k, rank):
    upb = f32_to_bf16_bits((rng.standard_normal((n, rank)) * 0.3).astype(np.float32))
    dnb = f32_to_bf16_bits((rng.standard_normal((k, rank)) * 0.3).astype(np.float32))
    return upb, dnb, O.bf16_decode(upb), O.bf16_decode(dnb)


def _split(w, rank, rng):
    n, k = w.shape
    if rank == 0:
        return None, None, np.zeros((n, 0)), np.zeros((k, 0))
    if n < rank:
        return _factors(rng, n, k, rank)
    up, dn = O.svd_init(w, rank)
    return bf16_bits_of(up), bf16_bits_of(dn), up, dn


# ------------------------------------------------------------------ quantizers
def test_mx_quantize_weight_shapes_and_ranks():
    import w4_gemm_amd as W
    rng = np.random.default_rng(31)
    for (n, k, rank) in [(100, 768, 32), (33, 256, 0), (64, 2048, 16), (200, 512, 64), (1, 1280, 16)]:
        w = gen_weight(rng, n, k, 4)
        upb, dnb, up, dn = _split(w, rank, rng)
        p, flags = W.quantize_weight_mx4(torch.from_numpy(w).to(dev()), _bf16_dev(upb), _bf16_dev(dnb))
        torch.cuda.synchronize()
        assert int(flags[0]) == 0
        r = O.residual(w, up, dn)
        rep = O.check_device_mx(r, O.mx_unpack(p.codes.cpu().numpy()), p.exps.cpu().numpy())
        print(f"n{n} k{k} r{rank}", rep)
        assert rep["ok"], rep


def test_mx_quantize_act():
    import w4_gemm_amd as W
    rng = np.random.default_rng(32)
    for (m, k) in [(1, 256), (17, 1024), (100, 3072), (64, 512)]:
        xbits = gen_activations(rng, m, k, 0.01)
        xbits[0, :] = 0                                    # an all-zero row
        if m > 2:
            xbits[1] = f32_to_bf16_bits(O.bf16_decode(xbits[1]).astype(np.float32) * 1e-20)
        xq, xs = W.quantize_act_mx4(_bf16_dev(xbits))
        torch.cuda.synchronize()
        a = O.rotate(O.bf16_decode(xbits))
        rep = O.check_device_mx(a, O.mx_unpack(xq.cpu().numpy()), xs.cpu().numpy())
        print(f"act m{m} k{k}", rep)
        assert rep["ok"], rep


def test_mx_quantize_flags():
    import w4_gemm_amd as W
    w = torch.zeros((16, 256), dtype=torch.float32, device=dev())
    w[2, 7] = float("inf")
    _, flags = W.quantize_weight_mx4(w, None, None)
    torch.cuda.synchronize()
    assert int(flags[0]) & 1


# ------------------------------------------------------------------ reconstruct
def _check_reconstruct(codes, exps, upb, dnb, tag, rows=None):
    import w4_gemm_amd as W
    n = codes.shape[0]
    k = codes.shape[1] * 2
    what = W.reconstruct_bf16_mx4(_payload(codes, exps, upb, dnb))
    torch.cuda.synchronize()
    rows = np.arange(n) if rows is None else rows
    got = bf16_tensor_to_f64(what[torch.from_numpy(rows).to(dev())])
    up = O.bf16_decode(upb[rows]) if upb is not None else np.zeros((len(rows), 0))
    dn = O.bf16_decode(dnb) if dnb is not None else np.zeros((k, 0))
    exact = O.reconstruct_mx(O.mx_unpack(codes[rows]), exps[rows], up, dn)
    ref = O.bf16_round(exact)
    e = O.rel_fro(got, ref)
    print(f"{tag}: reconstruct relF vs bf16(oracle) = {e:.3e}")
    assert e <= WHAT_TOL
    assert np.all(np.abs(got - ref) <= ulp_bf16(ref))


def test_mx_reconstruct_shapes_and_ranks():
    rng = np.random.default_rng(33)
    for (n, k, rank) in [(100, 768, 32), (33, 256, 0), (64, 2048, 16), (200, 512, 64), (17, 1024, 16)]:
        codes, exps, upb, dnb = gen_payload_mx(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        exps[0, 0] = 0                                     # a block at the smallest scale
        codes[1, :16] = 0                                  # an all-zero block
        _check_reconstruct(codes, exps, upb, dnb, f"n{n} k{k} r{rank}")


# ------------------------------------------------------------------ forward
def _fwd_checks(xbits, codes, exps, upb, dnb, rows=None, tag=""):
    import w4_gemm_amd as W
    k = codes.shape[1] * 2
    p = _payload(codes, exps, upb, dnb)
    xd = _bf16_dev(xbits)
    y32 = W.linear_fwd_mx4(xd, p, torch.float32)
    y16 = W.linear_fwd_mx4(xd, p, torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.arange(xbits.shape[0]) if rows is None else rows
    ri = torch.from_numpy(rows).to(dev())
    y32h = y32[ri].cpu().numpy().astype(np.float64)
    y16h = bf16_tensor_to_f64(y16[ri])
    assert np.all(np.isfinite(y32h))
    assert np.array_equal(y16h, O.bf16_round(y32h))
    x = O.bf16_decode(xbits[rows])
    up = O.bf16_decode(upb) if upb is not None else np.zeros((codes.shape[0], 0))
    dn = O.bf16_decode(dnb) if dnb is not None else np.zeros((k, 0))
    wc = O.mx_unpack(codes)
    ref = O.forward_mx(x, wc, exps, up, dn)
    e = O.rel_fro(y32h, ref)
    # rows whose rotated activations hold no value near a midpoint or a block
    # absmax near a power of two: the same FP4 operands on both sides
    a = O.rotate(x)
    ac, ae = O.mx_quantize(a)
    ok, near = O.certify_mx(a, ae)
    clean = ok.all(axis=1) & ~near.any(axis=1)
    num = np.linalg.norm(y32h - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    worst = float((num / den)[clean].max()) if clean.any() else 0.0
    # elsewhere: the deviation the admissible activation codes allow
    xs = np.repeat(np.ldexp(1.0, ae.astype(np.int64) - 127), O.MX_BLOCK, axis=1)
    delta = np.where(near, 2.0 * xs, 0.0)
    delta = np.maximum(delta, np.where(np.repeat(~ok, O.MX_BLOCK, axis=1), 4.0 * xs, 0.0))
    wd = np.abs(O.mx_dequant(wc, exps))
    bound = delta @ wd.T + ACC_TOL * (np.abs(O.mx_dequant(ac, ae)) @ wd.T
                                      + np.abs(x @ dn) @ np.abs(up).T) + 1e-30
    excess = float((np.abs(y32h - ref) / bound).max())
    print(f"{tag}: relF={e:.3e} clean rows {int(clean.sum())}/{len(rows)} "
          f"worst clean-row rel={worst:.3e} max |diff|/allowed={excess:.3f}")
    assert worst <= ROW_TOL and excess <= 1.0
    return y32h, ref


def test_mx_fwd_shapes():
    rng = np.random.default_rng(34)
    for (m, n, k, rank) in [(1, 200, 1280, 16), (17, 64, 2048, 32), (100, 300, 768, 0),
                            (257, 520, 1024, 64), (300, 33, 512, 16), (64, 256, 256, 32)]:
        codes, exps, upb, dnb = gen_payload_mx(rng, n, k, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, m, k, 0.01)
        _fwd_checks(xbits, codes, exps, upb, dnb, tag=f"m{m} n{n} k{k} r{rank}")


def test_mx_fwd_split_k():
    # grids of fewer than 128 tiles split K: 4 tiles x 8 splits of 8 stages,
    # 3 tiles x 3 splits of 8, 9 and 9 stages, 2 tiles x 5 splits of 9 or 10
    rng = np.random.default_rng(37)
    for (m, n, k, rank) in [(3, 1000, 8192, 32), (40, 513, 3328, 16), (256, 257, 5888, 64)]:
        codes, exps, upb, dnb = gen_payload_mx(rng, n, k, rank)
        xbits = gen_activations(rng, m, k, 0.01)
        _fwd_checks(xbits, codes, exps, upb, dnb, tag=f"split-K m{m} n{n} k{k} r{rank}")


def test_mx_end_to_end_quantized_layer():
    # device quantizer -> device forward; the FP4 layer tracks the exact layer
    import w4_gemm_amd as W
    rng = np.random.default_rng(35)
    n, k, m, rank = 192, 1024, 96, 32
    w = gen_weight(rng, n, k, 4)
    upb, dnb, up, dn = _split(w, rank, rng)
    p, flags = W.quantize_weight_mx4(torch.from_numpy(w).to(dev()), _bf16_dev(upb), _bf16_dev(dnb))
    torch.cuda.synchronize()
    codes, exps = p.codes.cpu().numpy(), p.exps.cpu().numpy()
    rep = O.check_device_mx(O.residual(w, up, dn), O.mx_unpack(codes), exps)
    assert rep["ok"], rep
    xbits = gen_activations(rng, m, k, 0.01)
    y, _ = _fwd_checks(xbits, codes, exps, upb, dnb, tag="e2e")
    x = O.bf16_decode(xbits)
    exact = x @ w.astype(np.float64).T
    cs = O.cosine(y, exact)
    print(f"e2e cosine vs the unquantized layer {cs:.5f}")
    assert cs > 0.99


def test_mx_full_size_sampled():
    # the MLP-up shape 4480 x 16384 x 6144, rank 32: whole layer on the GPU,
    # the oracle on sampled rows
    import w4_gemm_amd as W
    rng = np.random.default_rng(36)
    m, n, k, rank = 4480, 16384, 6144, 32
    codes, exps, upb, dnb = gen_payload_mx(rng, n, k, rank)
    xbits = gen_activations(rng, m, k, 0.005)
    rows = np.sort(rng.choice(m, 16, replace=False))
    _fwd_checks(xbits, codes, exps, upb, dnb, rows=rows, tag="full size")
    wr = np.sort(rng.choice(n, 48, replace=False))
    _check_reconstruct(codes, exps, upb, dnb, "full size", rows=wr)
