"""Device parity: libsq's HIP kernels against the CPU oracle.

Bars (from the layer's accuracy contract):
  * quantize: codes, fp16 scales and fraction indices bit-exact on every
    tie-certified group; uncertified groups must be admissible near-ties;
  * reconstruct: bf16 W_hat within 1e-3 relative Frobenius of the oracle's
    exact W_hat rounded to bf16, and at most 1 bf16 ulp per element;
  * forward: fp32 y within 2e-3 relative Frobenius (cos >= 0.9999) of the
    exact fp64 y; within 1e-5 of the oracle evaluated on the same fp16
    operands; bf16 y is bit-equal to round-to-nearest-even of the fp32 y.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, gen_layer, gen_payload
from tests.helpers import (bf16_bits_of, bf16_tensor_to_f64, dev, oracle_payload, payload_fp64,
                           to_dev_payload, ulp_bf16)

pytestmark = pytest.mark.gpu

Y_TOL, COS_TOL, DIAG_TOL, WHAT_TOL = 2e-3, 0.9999, 1e-5, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401  (fails loudly if libsq.so is missing)


def _x_dev(xbits):
    return torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(dev())


# ------------------------------------------------------------------ config 1, end to end
@pytest.fixture(scope="module")
def tiny():
    cfg, w, xbits = gen_layer(1, seed=0)
    codes, scales, upb, dnb, res, r, up, dn = oracle_payload(w, cfg.rank, cfg.group)
    return dict(cfg=cfg, w=w, xbits=xbits, codes=codes, scales=scales, upb=upb, dnb=dnb, res=res,
                r=r, up=up, dn=dn)


def _check_quant(w, up_bits, dn_bits, group, up, dn, tag):
    import w4_gemm_amd as W
    d = dev()
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(d)
    upt = torch.from_numpy(up_bits.view(np.int16)).view(torch.bfloat16).to(d) if up_bits is not None else None
    dnt = torch.from_numpy(dn_bits.view(np.int16)).view(torch.bfloat16).to(d) if dn_bits is not None else None
    p, fidx, flags = W.quantize_weight(wt, upt, dnt, group)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0
    r = O.residual(w, up, dn)
    res = O.quantize_residual(r, group)
    rep = O.check_device_quant(r, res, group, O.unpack(p.codes.cpu().numpy()),
                               p.scales.cpu().numpy().astype(np.float64), fidx.cpu().numpy())
    print(tag, rep)
    assert rep["ok"], rep
    return rep


def test_quantize_tiny(tiny):
    t = tiny
    _check_quant(t["w"], t["upb"], t["dnb"], 32, t["up"], t["dn"], "cfg1")


def test_quantize_tiny_g64_rank0_ragged():
    rng = np.random.default_rng(3)
    from synth import gen_weight
    w = gen_weight(rng, 100, 768, 4)            # N not a multiple of 16, three blocks
    up, dn = O.svd_init(w, 32)
    _check_quant(w, bf16_bits_of(up), bf16_bits_of(dn), 64, up, dn, "ragged g64")
    _check_quant(w, None, None, 32, np.zeros((100, 0)), np.zeros((768, 0)), "rank0 g32")


def test_quantize_edge_groups():
    # all-zero groups, grid-planted groups (exact), a negative-heavy group
    import w4_gemm_amd as W
    rng = np.random.default_rng(4)
    n, k, g = 16, 512, 32
    q = rng.integers(-7, 8, (n, k)); q[:, ::g] = 7
    s = O.fp16_round(rng.uniform(1e-3, 1e-2, (n, k // g)))
    r_plant = q * np.repeat(s, g, 1)
    w = O.rotate(r_plant)                                  # rank 0: W = R H
    w[3, :] = 0.0
    w32 = w.astype(np.float32)
    d = dev()
    p, fidx, flags = W.quantize_weight(torch.from_numpy(w32).to(d), None, None, g)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0
    qd = O.unpack(p.codes.cpu().numpy()); sd = p.scales.cpu().numpy().astype(np.float64)
    fd = fidx.cpu().numpy()
    assert np.all(qd[3] == 0) and np.all(sd[3] == 0) and np.all(fd[3] == 0)
    r = O.residual(w32, np.zeros((n, 0)), np.zeros((k, 0)))
    res = O.quantize_residual(r, g)
    rep = O.check_device_quant(r, res, g, qd, sd, fd)
    assert rep["ok"], rep


def test_quantize_flags():
    import w4_gemm_amd as W
    d = dev()
    w = torch.zeros((16, 256), dtype=torch.float32, device=d)
    w[2, 7] = float("nan")
    _, _, flags = W.quantize_weight(w, None, None, 32)
    torch.cuda.synchronize()
    assert int(flags[0]) & 1
    w = torch.zeros((16, 256), dtype=torch.float32, device=d)
    w[5, :] = 1e6                      # rotated values 1e6*16 -> absmax/7 > 65504
    _, _, flags = W.quantize_weight(w, None, None, 32)
    torch.cuda.synchronize()
    assert int(flags[0]) & 2


def test_reconstruct_tiny(tiny):
    import w4_gemm_amd as W
    t = tiny
    p = to_dev_payload(t["codes"], t["scales"], t["upb"], t["dnb"], 32)
    what = W.reconstruct_bf16(p)
    torch.cuda.synchronize()
    got = bf16_tensor_to_f64(what)
    q, s, up, dn = payload_fp64(t["codes"], t["scales"], t["upb"], t["dnb"])
    exact = O.reconstruct(q, s, up, dn, 32)
    ref = O.bf16_round(exact)
    assert O.rel_fro(got, ref) <= WHAT_TOL
    assert np.all(np.abs(got - ref) <= ulp_bf16(ref))
    assert O.cosine(got, exact) > 0.99999


@pytest.mark.parametrize("n,k,g,rank", [(100, 768, 64, 32), (16, 256, 64, 0), (33, 1024, 64, 64),
                                        (50, 512, 32, 0)])
def test_reconstruct_groups_ranks_ragged(n, k, g, rank):
    # every element, both group sizes, ranks 0/32/64, N ragged against the 16-row strips
    import w4_gemm_amd as W
    rng = np.random.default_rng(n + k + g)
    codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
    if rank == 0:
        upb = dnb = None
    p = to_dev_payload(codes, scales, upb, dnb, g)
    got = bf16_tensor_to_f64(W.reconstruct_bf16(p))
    torch.cuda.synchronize()
    q, s, up, dn = payload_fp64(codes, scales, upb, dnb)
    ref = O.bf16_round(O.reconstruct(q, s, up, dn, g))
    e = O.rel_fro(got, ref)
    print(f"reconstruct n{n} k{k} g{g} r{rank}: relF {e:.3e}")
    assert e <= WHAT_TOL and np.all(np.abs(got - ref) <= ulp_bf16(ref))


def _fwd_checks(xbits, codes, scales, upb, dnb, group, rows=None, tag=""):
    import w4_gemm_amd as W
    p = to_dev_payload(codes, scales, upb, dnb, group)
    xd = _x_dev(xbits)
    y32 = W.linear_fwd(xd, p, torch.float32)
    y16 = W.linear_fwd(xd, p, torch.bfloat16)
    torch.cuda.synchronize()
    y32h = y32.cpu().numpy().astype(np.float64)
    y16h = bf16_tensor_to_f64(y16)
    assert np.all(np.isfinite(y32h))
    # bf16 output is RNE of the fp32 output, bit for bit
    assert np.array_equal(y16h, O.bf16_round(y32h))
    rows = np.arange(xbits.shape[0]) if rows is None else rows
    x = O.bf16_decode(xbits[rows])
    q, s, up, dn = payload_fp64(codes, scales, upb, dnb)
    ref = O.forward(x, q, s, up, dn, group)
    diag = O.forward_fp16_operands(x, q, s, up, dn, group)
    got = y32h[rows]
    e, cs, ed = O.rel_fro(got, ref), O.cosine(got, ref), O.rel_fro(got, diag)
    print(f"{tag}: relF={e:.3e} cos={cs:.7f} vs-fp16-operands={ed:.3e}")
    assert e <= Y_TOL and cs >= COS_TOL and ed <= DIAG_TOL
    return y32h


def test_fwd_tiny(tiny):
    t = tiny
    _fwd_checks(t["xbits"], t["codes"], t["scales"], t["upb"], t["dnb"], 32, tag="cfg1")


def test_fwd_ragged_and_rank0():
    rng = np.random.default_rng(5)
    for (m, n, k, g, rank) in [(100, 200, 768, 64, 32), (3, 16, 256, 32, 0), (130, 33, 512, 32, 64)]:
        codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        from synth import gen_activations
        xbits = gen_activations(rng, m, k, 0.01)
        _fwd_checks(xbits, codes, scales, upb, dnb, g, tag=f"m{m} n{n} k{k} g{g} r{rank}")


def test_fwd_small_m_tiles():
    # the small-M contraction with one, two and four 16-row tiles and, above
    # 64 rows, two 64-row chunks (the second ragged); K slices that are and
    # are not whole multiples of its prefetch step; ragged N
    rng = np.random.default_rng(11)
    from synth import gen_activations
    for k in (1280, 2048):
        codes, scales, upb, dnb = gen_payload(rng, 200, k, 32, 32)
        xbits = gen_activations(rng, 128, k, 0.01)
        for m in (1, 17, 32, 33, 64, 65, 100, 128):
            _fwd_checks(xbits[:m], codes, scales, upb, dnb, 32, tag=f"m{m} n200 k{k}")


def test_fwd_mid_m_plans():
    # mid-size M with long K: the planner's picks here include 224- and
    # 256-row tiles with split-K and 224-row tiles without; M and N ragged
    rng = np.random.default_rng(12)
    from synth import gen_activations
    for (m, n, k, g, rank) in [(1500, 1540, 4096, 32, 32), (2000, 1800, 6144, 64, 64),
                               (2000, 4100, 1024, 32, 0)]:
        codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, m, k, 0.01)
        rows = np.sort(rng.choice(m, 24, replace=False))
        _fwd_checks(xbits, codes, scales, upb, dnb, g, rows=rows, tag=f"m{m} n{n} k{k} g{g} r{rank}")


def test_fwd_statistics_tile_plans():
    # long K and many rows: the statistics pass takes two, four and eight
    # 16-row tiles per workgroup (at rank 64 with two x tiles in flight, at
    # rank 32 with two and four), with a ragged last row tile; 4480 rows take
    # two tiles (eight would need more workgroups than fit at once)
    rng = np.random.default_rng(13)
    from synth import gen_activations
    for (m, n, k, rank) in [(1000, 256, 16384, 64), (2040, 300, 16384, 64), (1000, 256, 16384, 32),
                            (2040, 300, 16384, 32), (4470, 260, 16384, 64)]:
        codes, scales, upb, dnb = gen_payload(rng, n, k, 32, rank)
        xbits = gen_activations(rng, m, k, 0.01)
        rows = np.sort(np.concatenate([rng.choice(m - 1, 15, replace=False), [m - 1]]))
        _fwd_checks(xbits, codes, scales, upb, dnb, 32, rows=rows, tag=f"m{m} n{n} k{k} r{rank}")


def test_fwd_one_launch_prephase():
    # K <= 4096 at ranks 0 and 32 with M > 16: the statistics and rotation run
    # in one launch, a workgroup per 16-row strip whose eight waves take one or
    # two 256-column blocks each: one block in all (K = 256), nine (the first
    # wave two, the other seven one), sixteen (two each); M ragged against the
    # strips; the split rotate + contract calls give the one-call result bit
    # for bit
    import w4_gemm_amd as W
    rng = np.random.default_rng(14)
    from synth import gen_activations
    for (m, n, k, g, rank) in [(40, 96, 256, 32, 32), (33, 300, 2304, 64, 0),
                               (77, 128, 4096, 32, 32), (300, 260, 2304, 32, 32)]:
        codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, m, k, 0.01)
        _fwd_checks(xbits, codes, scales, upb, dnb, g, tag=f"m{m} n{n} k{k} g{g} r{rank}")
        p = to_dev_payload(codes, scales, upb, dnb, g)
        xd = _x_dev(xbits)
        ws = torch.empty(W.fwd_workspace_bytes(m, p), dtype=torch.uint8, device=dev())
        y1 = W.linear_fwd(xd, p, torch.float32, workspace=ws)
        y2 = torch.empty_like(y1)
        W.linear_fwd_rotate(xd, p, ws)
        W.linear_fwd_contract(m, p, y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)


def test_fwd_decode_shapes():
    # the M <= 16 path: K slices of 512 and 1024 values, whole and with a
    # one-block last slice; N ragged against its 256-row workgroups and its
    # 64-row waves; both group sizes; ranks 0, 32 and 64
    rng = np.random.default_rng(12)
    from synth import gen_activations
    for (n, k, g, rank) in [(200, 256, 32, 32), (300, 768, 64, 64), (256, 1280, 32, 0),
                            (520, 3328, 32, 32), (64, 2048, 64, 32), (1, 512, 32, 32)]:
        codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        xbits = gen_activations(rng, 16, k, 0.01)
        for m in (1, 2, 5, 16):
            _fwd_checks(xbits[:m], codes, scales, upb, dnb, g, tag=f"m{m} n{n} k{k} g{g} r{rank}")


def test_fwd_decode_split_calls_and_slices_apart():
    # rotate + contract on one workspace equals the one-call forward bit for
    # bit; a row whose K slices differ in scale by 1e8 keeps both (each slice
    # has its own power of two)
    import w4_gemm_amd as W
    rng = np.random.default_rng(13)
    codes, scales, upb, dnb = gen_payload(rng, 300, 2048, 32, 32)
    from synth import f32_to_bf16_bits
    x = rng.standard_normal((16, 2048)).astype(np.float32)
    x[3, :512] *= 1e4
    x[3, 512:] *= 1e-4
    x[5, 1024:] = 0.0
    xbits = f32_to_bf16_bits(x)
    p = to_dev_payload(codes, scales, upb, dnb, 32)
    for m in (1, 4, 16):
        _fwd_checks(xbits[:m], codes, scales, upb, dnb, 32, tag=f"slices apart m{m}")
        xd = _x_dev(xbits[:m])
        ws = torch.empty(W.fwd_workspace_bytes(m, p), dtype=torch.uint8, device=dev())
        y1 = W.linear_fwd(xd, p, torch.float32, workspace=ws)
        y2 = torch.empty_like(y1)
        W.linear_fwd_rotate(xd, p, ws)
        W.linear_fwd_contract(m, p, y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)


def test_fwd_zero_rows_and_large_activations():
    import w4_gemm_amd as W
    rng = np.random.default_rng(6)
    codes, scales, upb, dnb = gen_payload(rng, 64, 512, 32, 32)
    from synth import f32_to_bf16_bits
    x = rng.standard_normal((20, 512)).astype(np.float32)
    x[4] = 0.0                                       # an all-zero row
    x[7] *= 3.0e4                                    # far outside fp16 range after rotation
    x[9] *= 1e-30                                    # tiny row
    _fwd_checks(f32_to_bf16_bits(x), codes, scales, upb, dnb, 32, tag="edge rows")
    # m == 0 is a no-op
    p = to_dev_payload(codes, scales, upb, dnb, 32)
    y = torch.empty((0, 64), device=dev())
    W.linear_fwd(torch.empty((0, 512), dtype=torch.bfloat16, device=dev()), p, out=y)


def test_determinism(tiny):
    import w4_gemm_amd as W
    t = tiny
    p = to_dev_payload(t["codes"], t["scales"], t["upb"], t["dnb"], 32)
    xd = _x_dev(t["xbits"])
    a = W.linear_fwd(xd, p); b = W.linear_fwd(xd, p)
    ra = W.reconstruct_bf16(p); rb = W.reconstruct_bf16(p)
    wt = torch.from_numpy(t["w"]).to(dev())
    q1, f1, _ = W.quantize_weight(wt, p.up, p.down, 32)
    q2, f2, _ = W.quantize_weight(wt, p.up, p.down, 32)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ra.view(torch.int16), rb.view(torch.int16))
    assert torch.equal(q1.codes, q2.codes) and torch.equal(f1, f2)
    assert torch.equal(q1.scales.view(torch.int16), q2.scales.view(torch.int16))


# ------------------------------------------------------------------ input gradient
def _dgrad_checks(dybits, codes, scales, upb, dnb, group, rows=None, tag=""):
    import w4_gemm_amd as W
    p = to_dev_payload(codes, scales, upb, dnb, group)
    dyd = _x_dev(dybits)
    d32 = W.linear_dgrad(dyd, p, torch.float32)
    d16 = W.linear_dgrad(dyd, p, torch.bfloat16)
    torch.cuda.synchronize()
    d32h = d32.cpu().numpy().astype(np.float64)
    d16h = bf16_tensor_to_f64(d16)
    assert np.all(np.isfinite(d32h))
    assert np.array_equal(d16h, O.bf16_round(d32h))
    rows = np.arange(dybits.shape[0]) if rows is None else rows
    dy = O.bf16_decode(dybits[rows])
    q, s, up, dn = payload_fp64(codes, scales, upb, dnb)
    ref = O.dgrad(dy, q, s, up, dn, group)
    diag = O.dgrad_fp16_operands(dy, q, s, up, dn, group)
    got = d32h[rows]
    e, cs, ed = O.rel_fro(got, ref), O.cosine(got, ref), O.rel_fro(got, diag)
    print(f"{tag}: dgrad relF={e:.3e} cos={cs:.7f} vs-fp16-operands={ed:.3e}")
    assert e <= Y_TOL and cs >= COS_TOL and ed <= DIAG_TOL
    return d32h


def _gen_dy(rng, m, n):
    from synth import f32_to_bf16_bits
    dy = rng.standard_normal((m, n)).astype(np.float32)
    if m > 4:
        dy[1] = 0.0                # an all-zero row
        dy[2] *= 1e-6              # a small-gradient row (the fp16 row factor matters)
        dy[3] *= 3.0e4             # a large one
    return f32_to_bf16_bits(dy)


def test_dgrad_tiny(tiny):
    t = tiny
    dyb = _gen_dy(np.random.default_rng(21), t["cfg"].M, t["cfg"].N)
    _dgrad_checks(dyb, t["codes"], t["scales"], t["upb"], t["dnb"], 32, tag="cfg1")


def test_dgrad_ragged_ranks_groups():
    # N not a multiple of 256 (the input gradient's own statistics kernel) and
    # N a multiple of 256 (the statistics kernel it shares with the forward)
    rng = np.random.default_rng(22)
    for (m, n, k, g, rank) in [(100, 192, 768, 64, 32), (3, 64, 256, 32, 0), (130, 128, 512, 32, 64),
                               (257, 320, 1024, 64, 32), (257, 512, 1024, 32, 64),
                               (100, 256, 768, 64, 0), (50, 768, 512, 32, 32)]:
        codes, scales, upb, dnb = gen_payload(rng, n, k, g, max(rank, 1))
        if rank == 0:
            upb = dnb = None
        _dgrad_checks(_gen_dy(rng, m, n), codes, scales, upb, dnb, g,
                      tag=f"m{m} n{n} k{k} g{g} r{rank}")


def test_dgrad_determinism_and_empty(tiny):
    import w4_gemm_amd as W
    t = tiny
    p = to_dev_payload(t["codes"], t["scales"], t["upb"], t["dnb"], 32)
    dyd = _x_dev(_gen_dy(np.random.default_rng(23), 64, t["cfg"].N))
    a = W.linear_dgrad(dyd, p); b = W.linear_dgrad(dyd, p)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    W.linear_dgrad(torch.empty((0, t["cfg"].N), dtype=torch.bfloat16, device=dev()), p,
                   out=torch.empty((0, t["cfg"].K), device=dev()))


@pytest.mark.parametrize("cfg_id", [2, 4, 5])
def test_dgrad_full_size_sampled(cfg_id):
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng(300 + cfg_id)
    codes, scales, upb, dnb = gen_payload(rng, cfg.N, cfg.K, cfg.group, cfg.rank)
    dyb = _gen_dy(np.random.default_rng(cfg_id), cfg.M, cfg.N)
    rows = np.sort(np.concatenate([[1, 2, 3], np.random.default_rng(7).choice(
        np.arange(4, cfg.M), 21, replace=False)]))
    _dgrad_checks(dyb, codes, scales, upb, dnb, cfg.group, rows=rows, tag=f"cfg{cfg_id}")


# ------------------------------------------------------------------ full-size shapes
@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5])
def test_fwd_full_size_sampled(cfg_id):
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng(100 + cfg_id)
    codes, scales, upb, dnb = gen_payload(rng, cfg.N, cfg.K, cfg.group, cfg.rank)
    from synth import gen_activations
    xbits = gen_activations(np.random.default_rng(cfg_id), cfg.M, cfg.K, cfg.outlier_frac)
    rows = np.sort(np.random.default_rng(7).choice(cfg.M, 24, replace=False))
    _fwd_checks(xbits, codes, scales, upb, dnb, cfg.group, rows=rows, tag=f"cfg{cfg_id}")
    if cfg.small_m:
        for m in cfg.small_m:
            _fwd_checks(xbits[:m], codes, scales, upb, dnb, cfg.group,
                        rows=np.arange(min(m, 16)), tag=f"cfg{cfg_id} M={m}")


@pytest.mark.parametrize("cfg_id", [2, 4, 5])
def test_reconstruct_full_size_sampled(cfg_id):
    import w4_gemm_amd as W
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng(200 + cfg_id)
    codes, scales, upb, dnb = gen_payload(rng, cfg.N, cfg.K, cfg.group, cfg.rank)
    p = to_dev_payload(codes, scales, upb, dnb, cfg.group)
    what = W.reconstruct_bf16(p)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(8).choice(cfg.N, 48, replace=False))
    got = bf16_tensor_to_f64(what[torch.from_numpy(rows).to(dev())])
    q, s, up, dn = payload_fp64(codes[rows], scales[rows], upb[rows], dnb)
    exact = O.reconstruct(q, s, up, dn, cfg.group)
    ref = O.bf16_round(exact)
    e = O.rel_fro(got, ref)
    print(f"cfg{cfg_id} reconstruct relF vs bf16(oracle) = {e:.3e}")
    assert e <= WHAT_TOL
    assert np.all(np.abs(got - ref) <= ulp_bf16(ref))


def test_quantize_cfg3_sampled_rows():
    # the fused-QKV weight (9216 x 3072, g64): whole weight on the GPU, oracle on sampled rows
    cfg, w, _ = gen_layer(3, seed=0, with_x=False)
    up, dn = O.svd_init(w, cfg.rank)
    rows = np.sort(np.random.default_rng(9).choice(cfg.N, 192, replace=False))
    import w4_gemm_amd as W
    d = dev()
    p, fidx, flags = W.quantize_weight(torch.from_numpy(w).to(d),
                                       torch.from_numpy(bf16_bits_of(up).view(np.int16)).view(torch.bfloat16).to(d),
                                       torch.from_numpy(bf16_bits_of(dn).view(np.int16)).view(torch.bfloat16).to(d),
                                       cfg.group)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0
    r = O.residual(w[rows], up[rows], dn)
    res = O.quantize_residual(r, cfg.group)
    rep = O.check_device_quant(r, res, cfg.group, O.unpack(p.codes[torch.from_numpy(rows).to(d)].cpu().numpy()),
                               p.scales[torch.from_numpy(rows).to(d)].cpu().numpy().astype(np.float64),
                               fidx[torch.from_numpy(rows).to(d)].cpu().numpy())
    print("cfg3 quantize", rep)
    assert rep["ok"], rep


# ------------------------------------------------------------------ fp16 range of the operands
def _edge_scale_payload(rng, n=64, k=512, g=32, rank=32):
    """Rows in four bands of scales: 8188 (the largest with 8 s <= 65504, with
    code -8 present), 2^-20 (fp16 subnormal), 2^-14 (smallest normal), 1e-3."""
    q = rng.integers(-8, 8, (n, k))
    q[:16, ::g] = -8
    bands = [8188.0, 2.0 ** -20, 2.0 ** -14, float(np.float16(1e-3))]
    s = np.repeat(np.array(bands), n // 4)[:, None] * np.ones((1, k // g))
    codes = O.pack(q)
    scales = s.astype(np.float16)
    up = bf16_bits_of(O.bf16_round(rng.standard_normal((n, rank)) * 0.1))
    dn = bf16_bits_of(O.bf16_round(rng.standard_normal((k, rank)) * 0.1))
    return codes, scales, up, dn


def test_fwd_and_dgrad_at_scale_range_edges():
    rng = np.random.default_rng(31)
    codes, scales, upb, dnb = _edge_scale_payload(rng)
    from synth import gen_activations
    for m in (3, 40, 200):
        xbits = gen_activations(rng, m, 512, 0.01)
        _fwd_checks(xbits, codes, scales, upb, dnb, 32, tag=f"scale edges m{m}")
        _dgrad_checks(_gen_dy(rng, m, 64), codes, scales, upb, dnb, 32, tag=f"scale edges m{m}")


def test_quantize_fp16_range_flag():
    import w4_gemm_amd as W
    rng = np.random.default_rng(32)
    n, k, g = 16, 512, 32
    q = rng.integers(-7, 8, (n, k)); q[:, ::g] = 7
    d = dev()
    for s, want in ((8188.0, 0), (9000.0, 4)):
        w = O.rotate(q * s).astype(np.float32)            # rank 0, grid-planted: f = 1.00 exact
        p, fidx, flags = W.quantize_weight(torch.from_numpy(w).to(d), None, None, g)
        torch.cuda.synchronize()
        assert int(flags[0]) == want, (s, int(flags[0]))
        assert np.all(p.scales.cpu().numpy().astype(np.float64) == s)
        # the reconstruct (fp32) is exact for either payload
        what = bf16_tensor_to_f64(W.reconstruct_bf16(p))
        assert np.array_equal(what, O.bf16_round(O.rotate(q * s)))
