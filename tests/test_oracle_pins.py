"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a textbook or library
routine, exact rational arithmetic or an invariant of the method (SquareQ
README, "SquareQ v3 - W4" section).  ``test_planted_mistakes`` at the end
plants plausible mistakes in the oracle and shows a pin here catches each.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O
from synth import f32_to_bf16_bits, bf16_bits_to_f32


# ----------------------------------------------------------------- Hadamard
def pin_sylvester_matches_kronecker():
    # textbook recursion S_2n = [[S, S], [S, -S]], independent of popcount
    s = np.array([[1.0]])
    while s.shape[0] < 256:
        s = np.block([[s, s], [s, -s]])
    assert np.array_equal(O.sylvester(256), s)
    # and the library's Sylvester construction
    assert np.array_equal(O.sylvester(256), scipy.linalg.hadamard(256).astype(float))


def pin_hadamard_orthonormal_selfinverse():
    h = O.hadamard256()
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, np.eye(256))           # exact: sums of +-1/256


def pin_rotate_blocks():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 768))
    r = O.rotate(x)
    # block-diagonal: each 256-block transforms on its own, H applied on the right
    h = scipy.linalg.hadamard(256) / 16.0
    for b in range(3):
        np.testing.assert_allclose(r[:, 256 * b:256 * b + 256], x[:, 256 * b:256 * b + 256] @ h,
                                   rtol=0, atol=1e-13)
    np.testing.assert_allclose(r, O.fwht_fast(x), rtol=0, atol=1e-13)
    # self-inverse and Parseval per block
    np.testing.assert_allclose(O.rotate(r), x, rtol=0, atol=1e-13)
    np.testing.assert_allclose((r.reshape(5, 3, 256) ** 2).sum(-1),
                               (x.reshape(5, 3, 256) ** 2).sum(-1), rtol=1e-13)
    # unit vectors: e0 -> 1/16 * ones ; ones -> 16 * e0
    e0 = np.zeros((1, 256)); e0[0, 0] = 1
    assert np.array_equal(O.rotate(e0), np.full((1, 256), 1 / 16))
    assert np.array_equal(O.rotate(np.ones((1, 256))), 16 * e0)
    # e_j -> row j of H: sign pattern (-1)^popcount(j & i)
    ej = np.zeros((1, 256)); ej[0, 37] = 1
    expect = np.array([(-1) ** bin(37 & i).count("1") for i in range(256)]) / 16
    assert np.array_equal(O.rotate(ej)[0], expect)


# ----------------------------------------------------------------- formats
def pin_fp16_round_matches_ieee():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        # exact ties between neighbours (round to even)
        (np.arange(1, 2000) * 2 + 1) * 2.0 ** -11 + 1.0,
        [65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 1e-9, 0.0],
    ])
    ours = O.fp16_round(v)
    with np.errstate(over="ignore"):
        lib = v.astype(np.float16).astype(np.float64)   # numpy rounds fp64 -> fp16 correctly
    assert np.array_equal(ours, lib, equal_nan=True)


def pin_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    v32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    ties = (1.0 + (np.arange(1, 500) * 2 + 1) * 2.0 ** -8).astype(np.float32)
    v32 = np.concatenate([v32, ties, -ties])
    ours = O.bf16_round(v32.astype(np.float64))
    lib = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, lib)
    # the generator's bit encoding agrees too (fp32 inputs)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(v32)).astype(np.float64), ours)


def pin_bf16_no_double_rounding():
    # x just above a bf16 tie: fp32 would round it onto the tie, fp64 -> bf16 must not
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40          # tie at 1 + 2^-8 between 1 and 1 + 2^-7
    assert O.bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7


# ----------------------------------------------------------------- SVD split
def pin_svd_split():
    rng = np.random.default_rng(4)
    n, k, r = 96, 80, 6
    u = np.linalg.qr(rng.standard_normal((n, r)))[0]
    v = np.linalg.qr(rng.standard_normal((k, r)))[0]
    sig = np.array([9.0, 7, 5, 3, 2, 1])
    w = (u * sig) @ v.T
    up, dn = O.svd_init(w, r, round_bf16=False)
    np.testing.assert_allclose(up @ dn.T, w, atol=1e-12)          # exact at full rank
    up, dn = O.svd_init(w, 32)                                    # rank > true rank: zero tail
    assert up.shape == (n, 32) and dn.shape == (k, 32)
    assert O.rel_fro(up @ dn.T, w) < 8e-3                         # only bf16 rounding left
    # Eckart-Young on a generic matrix
    w2 = rng.standard_normal((64, 48))
    s = np.linalg.svd(w2, compute_uv=False)
    for rank in (1, 5, 20):
        up, dn = O.svd_init(w2, rank, round_bf16=False)
        err = ((w2 - up @ dn.T) ** 2).sum()
        assert abs(err - (s[rank:] ** 2).sum()) < 1e-9 * (s ** 2).sum()
    # bf16 factors: every entry is a bf16 value
    up, dn = O.svd_init(w2, 8)
    assert np.array_equal(O.bf16_round(up), up) and np.array_equal(O.bf16_round(dn), dn)


def pin_spike_recovered():
    from synth import gen_weight
    rng = np.random.default_rng(5)
    w = gen_weight(rng, 512, 512, 4).astype(np.float64)
    s = np.linalg.svd(w, compute_uv=False)
    # planted singular values 8..2 dominate the N(0,1/K) bulk (edge ~ 2)
    np.testing.assert_allclose(s[:3], [8, 6, 4], rtol=0.1)


# ----------------------------------------------------------------- sweep
def _fp16_round_exact(v: Fraction) -> Fraction:
    """IEEE binary16 RNE of a non-negative rational, in exact arithmetic."""
    if v == 0:
        return Fraction(0)
    e = 0
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    e = max(e, -14)
    spacing = Fraction(2) ** (e - 10)
    n = v / spacing
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * spacing
    assert out <= 65504
    return out


def _rint_half_even(t: Fraction) -> int:
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _sweep_exact(r):
    """Brute-force sweep of one group in exact rational arithmetic."""
    rf = [Fraction(x) for x in r]
    a = max(abs(x) for x in rf)
    best = None
    for i in range(31):
        s = _fp16_round_exact(Fraction(70 + i, 700) * a)
        q = [0 if s == 0 else min(7, max(-8, _rint_half_even(x / s))) for x in rf]
        e = sum((x - qq * s) ** 2 for x, qq in zip(rf, q))
        if best is None or e < best[0]:
            best = (e, i, s, q)
    return best


def pin_sweep_exact_rational():
    rng = np.random.default_rng(6)
    groups = []
    for g in (32, 64):
        for _ in range(12):
            # dyadic values so the fp64 oracle's inputs are exact
            r = rng.integers(-4000, 4001, g) * 2.0 ** -14
            groups.append(r)
        # groups whose absmax is negative (the asymmetric -8 side)
        r = rng.integers(-300, 301, g) * 2.0 ** -12
        r[3] = -1000 * 2.0 ** -12
        groups.append(r)
        # heavy tails
        r = np.round(rng.standard_t(2, g) * 256) * 2.0 ** -10
        groups.append(r)
        # exact half-integer ties at the winning scale (f = 1.00, s = 100 * 2^-10):
        # values on that grid with large codes plus one or two half-way values,
        # so the rounding rule decides the emitted codes
        for _ in range(4):
            kk = rng.choice([-7, -6, -5, -4, 4, 5, 6, 7], g).astype(float)
            kk[0] = 7
            kk[1:3] = rng.choice([-1.5, -0.5, 0.5, 1.5, 2.5], 2)
            groups.append(kk * 100 * 2.0 ** -10)
    for r in groups:
        g = len(r)
        res = O.quantize_residual(np.tile(r, 256 // g)[None, :], g)
        e, i, s, q = _sweep_exact(r)
        assert res.fidx[0, 0] == i
        assert res.scale[0, 0] == float(s)
        assert np.array_equal(res.q[0, :g], np.array(q))
        assert abs(res.mse[0, 0, i] - float(e)) <= 1e-12 * max(float(e), 1e-30)


def pin_grid_planted():
    rng = np.random.default_rng(7)
    for g in (32, 64):
        n, k = 8, 512
        q = rng.integers(-7, 8, (n, k))
        q[:, ::g] = 7 * rng.choice([-1, 1], (n, k // g))            # |q| = 7 in every group
        s = O.fp16_round(rng.uniform(1e-3, 3e-2, (n, k // g)))
        r = q * np.repeat(s, g, axis=1)
        res = O.quantize_residual(r, g)
        assert np.array_equal(res.q, q)
        assert np.array_equal(res.scale, s)
        assert np.all(res.fidx == 30)
        best = np.take_along_axis(res.mse, res.fidx[..., None].astype(int), 2)[..., 0]
        assert np.all(best == 0)


def pin_sweep_invariances():
    rng = np.random.default_rng(8)
    r = rng.standard_normal((6, 512)) * 0.01
    base = O.quantize_residual(r, 32)
    for k in (-3, 4):
        sc = O.quantize_residual(r * 2.0 ** k, 32)
        assert np.array_equal(sc.q, base.q) and np.array_equal(sc.fidx, base.fidx)
        assert np.array_equal(sc.scale, base.scale * 2.0 ** k)
    # permuting whole groups permutes the result
    perm = rng.permutation(16)
    rp = r.reshape(6, 16, 32)[:, perm].reshape(6, 512)
    pp = O.quantize_residual(rp, 32)
    assert np.array_equal(pp.fidx, base.fidx[:, perm])
    assert np.array_equal(pp.q.reshape(6, 16, 32), base.q.reshape(6, 16, 32)[:, perm])
    # the chosen error never exceeds plain round-to-nearest at f = 1.00
    best = np.take_along_axis(base.mse, base.fidx[..., None].astype(int), 2)[..., 0]
    assert np.all(best <= base.mse[..., 30])
    # all-zero group: scale 0, codes 0, index 0
    z = r.copy(); z[2, 64:96] = 0
    zr = O.quantize_residual(z, 32)
    assert zr.fidx[2, 2] == 0 and zr.scale[2, 2] == 0 and np.all(zr.q[2, 64:96] == 0)
    # codes stay in range; the -8 code is reachable
    assert base.q.min() >= -8 and base.q.max() <= 7
    neg = np.zeros((1, 256)); neg[0, :32] = np.linspace(-1, 0.5, 32) * 0.01
    assert O.quantize_residual(neg, 32).q.min() == -8


def pin_non_finite_raises():
    r = np.zeros((1, 256)); r[0, 5] = np.nan
    with pytest.raises(FloatingPointError):
        O.quantize_residual(r, 32)
    r = np.zeros((1, 256)); r[0, 5] = 1e6                   # a/7 > 65504
    with pytest.raises(FloatingPointError):
        O.quantize_residual(r, 32)


# ----------------------------------------------------------------- packing
def pin_pack():
    assert list(O.pack(np.array([[1, -1, -8, 7]]))[0]) == [0xF1, 0x78]
    allbytes = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(O.pack(O.unpack(allbytes)), allbytes)
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]])
    assert np.array_equal(O.unpack(O.pack(q)), q)


# ----------------------------------------------------------------- the layer
def _payload(rng, n, k, g, rank):
    q = rng.integers(-8, 8, (n, k))
    s = O.fp16_round(rng.uniform(1e-3, 1e-2, (n, k // g)))
    up = O.bf16_round(rng.standard_normal((n, rank)) * 0.1)
    dn = O.bf16_round(rng.standard_normal((k, rank)) * 0.1)
    return q, s, up, dn


def pin_reconstruct_roundtrip():
    rng = np.random.default_rng(9)
    n, k, g = 16, 512, 32
    q = rng.integers(-7, 8, (n, k)); q[:, ::g] = 7
    s = O.fp16_round(rng.uniform(1e-3, 1e-2, (n, k // g)))
    up = O.bf16_round(rng.standard_normal((n, 32)) * 0.1)
    dn = O.bf16_round(rng.standard_normal((k, 32)) * 0.1)
    w = up @ dn.T + O.rotate(q * np.repeat(s, g, 1))      # a weight on the W4 grid
    res = O.quantize_weight(w, up, dn, g)
    assert np.array_equal(res.q, q) and np.array_equal(res.scale, s) and np.all(res.fidx == 30)
    np.testing.assert_allclose(O.reconstruct(res.q, res.scale, up, dn, g), w, rtol=0, atol=1e-15)


def pin_forward_consistent():
    rng = np.random.default_rng(10)
    n, k, g, m = 24, 512, 64, 7
    q, s, up, dn = _payload(rng, n, k, g, 32)
    x = O.bf16_round(rng.standard_normal((m, k)))
    y = O.forward(x, q, s, up, dn, g)
    what = O.reconstruct(q, s, up, dn, g)
    np.testing.assert_allclose(y, x @ what.T, rtol=1e-12, atol=1e-13)
    # linearity in x
    x2 = O.bf16_round(rng.standard_normal((m, k)))
    np.testing.assert_allclose(O.forward(x + 2 * x2, q, s, up, dn, g),
                               y + 2 * O.forward(x2, q, s, up, dn, g), atol=1e-12)
    # rank 0: a rotated int4 GEMM
    y0 = O.forward(x, q, s, up[:, :0], dn[:, :0], g)
    d = q * np.repeat(s, g, 1)
    np.testing.assert_allclose(y0, x @ O.rotate(d).T, atol=1e-12)
    # diagnostic fp16-operand forward: equal when every operand is fp16-exact
    xi = rng.integers(-3, 4, (m, k)).astype(float) * 16     # rotate(x) lands on small integers/16
    qi = rng.integers(-8, 8, (n, k)); si = np.full((n, k // g), 2.0 ** -7)
    np.testing.assert_allclose(O.forward_fp16_operands(xi, qi, si, up, dn, g),
                               O.forward(xi, qi, si, up, dn, g), rtol=1e-12, atol=1e-12)
    # and close (fp16 rounding) in general, also with large activations
    yd = O.forward_fp16_operands(x * 3000, q, s, up, dn, g)
    assert np.all(np.isfinite(yd))
    assert O.rel_fro(yd, O.forward(x * 3000, q, s, up, dn, g)) < 2e-3


def pin_dgrad_adjoint():
    # the input gradient is the adjoint of the forward: <dy, f(x)> = <g(dy), x>
    # for every x and dy, and it equals dy @ W_hat built explicitly
    rng = np.random.default_rng(14)
    n, k, g, m = 40, 768, 32, 5
    q, s, up, dn = _payload(rng, n, k, g, 32)
    x = rng.standard_normal((m, k))
    dy = rng.standard_normal((m, n))
    dx = O.dgrad(dy, q, s, up, dn, g)
    lhs = np.sum(dy * O.forward(x, q, s, up, dn, g))
    rhs = np.sum(dx * x)
    assert abs(lhs - rhs) <= 1e-12 * np.linalg.norm(dy) * np.linalg.norm(x) * np.linalg.norm(
        O.reconstruct(q, s, up, dn, g))
    np.testing.assert_allclose(dx, dy @ O.reconstruct(q, s, up, dn, g), rtol=1e-12, atol=1e-13)
    # one output feature, one K block, rank 0: dx is that weight row scaled
    e = np.zeros((1, n)); e[0, 3] = 2.0
    row = O.dgrad(e, q, s, up[:, :0], dn[:, :0], g)
    w0 = O.rotate(q[3:4] * np.repeat(s[3:4], g, 1))
    np.testing.assert_allclose(row, 2.0 * w0, atol=1e-14)
    # fp16-operand diagnostic: exact on fp16-exact operands, close otherwise
    dyi = rng.integers(-3, 4, (m, n)).astype(float)
    si = np.full((n, k // g), 2.0 ** -7)
    np.testing.assert_allclose(O.dgrad_fp16_operands(dyi, q, si, up, dn, g),
                               O.dgrad(dyi, q, si, up, dn, g), rtol=1e-12, atol=1e-12)
    dd = O.dgrad_fp16_operands(dy * 1e-6, q, s, up, dn, g)
    assert O.rel_fro(dd, O.dgrad(dy * 1e-6, q, s, up, dn, g)) < 2e-3


def pin_low_rank_weight():
    rng = np.random.default_rng(11)
    n, k = 128, 512
    u = np.linalg.qr(rng.standard_normal((n, 8)))[0]
    v = np.linalg.qr(rng.standard_normal((k, 8)))[0]
    w = (u * np.linspace(8, 2, 8)) @ v.T
    up, dn = O.svd_init(w, 32)
    r = O.residual(w, up, dn)
    assert np.linalg.norm(r) < 1e-2 * np.linalg.norm(w)       # only bf16 rounding remains


def pin_group_granularity():
    # finer groups fit better on average (a statistical, not per-instance, property)
    rng = np.random.default_rng(12)
    r = rng.standard_normal((64, 1024)) / 32
    e = {}
    for g in (32, 64):
        res = O.quantize_residual(r, g)
        e[g] = O.rel_fro(O.dequant(res.q, res.scale, g), r)
    assert e[32] < e[64] < 0.2


def pin_certification():
    rng = np.random.default_rng(13)
    r = rng.standard_normal((64, 512)) * 0.01
    res = O.quantize_residual(r, 32)
    rep = O.check_device_quant(r, res, 32, res.q, res.scale, res.fidx)
    assert rep["ok"] and rep["differ"] == 0
    cert = O.certify(r, res, 32)
    assert cert.mean() > 0.8
    # flipping a code in a certified group is caught
    gi = np.argwhere(cert)[0]
    qd = res.q.copy()
    qd[gi[0], gi[1] * 32] = (qd[gi[0], gi[1] * 32] + 1) if qd[gi[0], gi[1] * 32] < 7 else 6
    assert not O.check_device_quant(r, res, 32, qd, res.scale, res.fidx)["ok"]
    # a wrong index with its own consistent scale/codes is caught too
    fd = res.fidx.copy(); fd[gi[0], gi[1]] = (fd[gi[0], gi[1]] + 5) % 31
    sd = res.scale.copy()
    sd[gi[0], gi[1]] = O.fp16_round(O.candidate_scale_exact(res.absmax[gi[0], gi[1]], fd[gi[0], gi[1]]))
    qd = res.q.copy()
    seg = slice(gi[1] * 32, gi[1] * 32 + 32)
    qd[gi[0], seg] = O.codes_for_scale(r[gi[0], seg], sd[gi[0], gi[1]])
    assert not O.check_device_quant(r, res, 32, qd, sd, fd)["ok"]
    # the chosen scale rounded the other way: admissible only at a scale near-tie
    S = O.sq_oracle
    v = O.candidate_scale_exact(res.absmax, res.fidx)
    marg = S._fp16_boundary_margin(v)
    lo, hi = S._fp16_bracket(v)
    other = np.where(res.scale == lo, hi, lo)
    for want_ok, pick in ((True, np.argwhere(marg <= S.SCALE_MARGIN)[0]),
                          (False, np.argwhere(cert & (marg > 1e-4))[0])):
        i, g = pick
        sd = res.scale.copy(); sd[i, g] = other[i, g]
        qd = res.q.copy()
        seg = slice(g * 32, g * 32 + 32)
        qd[i, seg] = O.codes_for_scale(r[i, seg], sd[i, g])
        assert O.check_device_quant(r, res, 32, qd, sd, res.fidx)["ok"] == want_ok


# ----------------------------------------------------------------- int8-residual mode
def _sweep_exact_w8(r):
    """Brute-force row sweep of the int8 mode in exact rational arithmetic."""
    rf = [Fraction(x) for x in r]
    a = max(abs(x) for x in rf)
    best = None
    for i in range(31):
        s = _fp16_round_exact(Fraction(70 + i, 12700) * a)
        q = [0 if s == 0 else min(127, max(-128, _rint_half_even(x / s))) for x in rf]
        e = sum((x - qq * s) ** 2 for x, qq in zip(rf, q))
        if best is None or e < best[0]:
            best = (e, i, s, q)
    return best


def pin_w8_sweep_exact_rational():
    rng = np.random.default_rng(21)
    rows = []
    for _ in range(6):
        rows.append(rng.integers(-60000, 60001, 256) * 2.0 ** -20)        # dyadic, exact in fp64
    r = rng.integers(-3000, 3001, 256) * 2.0 ** -16
    r[7] = -9000 * 2.0 ** -16                                             # absmax on the -128 side
    rows.append(r)
    rows.append(np.round(rng.standard_t(2, 256) * 512) * 2.0 ** -12)      # heavy tails
    # exact half-integer ties at the winning scale (f = 1.00, s = 127 * 2^-12)
    for _ in range(3):
        kk = rng.integers(-127, 128, 256).astype(float)
        kk[0] = 127
        kk[1:4] = rng.choice([-100.5, -0.5, 0.5, 2.5, 63.5], 3)
        rows.append(kk * 127 * 2.0 ** -12 / 127)
    for r in rows:
        res = O.quantize_residual_w8(r[None, :])
        e, i, s, q = _sweep_exact_w8(r)
        assert res.fidx[0] == i
        assert res.scale[0] == float(s)
        assert np.array_equal(res.q[0], np.array(q))
        assert abs(res.mse[0, i] - float(e)) <= 1e-12 * max(float(e), 1e-30)


def pin_w8_grid_planted():
    rng = np.random.default_rng(22)
    n, k = 6, 768
    q = rng.integers(-127, 128, (n, k))
    q[:, 5] = 127 * rng.choice([-1, 1], n)                                # |q| = 127 in every row
    s = O.fp16_round(rng.uniform(1e-4, 3e-3, n))
    res = O.quantize_residual_w8(q * s[:, None])
    assert np.array_equal(res.q, q) and np.array_equal(res.scale, s)
    assert np.all(res.fidx == 30) and np.all(res.mse[np.arange(n), 30] == 0)


def pin_w8_invariances():
    rng = np.random.default_rng(23)
    r = rng.standard_normal((5, 512)) * 0.02
    base = O.quantize_residual_w8(r)
    for k in (-2, 5):
        sc = O.quantize_residual_w8(r * 2.0 ** k)
        assert np.array_equal(sc.q, base.q) and np.array_equal(sc.fidx, base.fidx)
        assert np.array_equal(sc.scale, base.scale * 2.0 ** k)
    # a per-row scale: permuting values within a row permutes the codes only
    perm = rng.permutation(512)
    pr = O.quantize_residual_w8(r[:, perm])
    assert np.array_equal(pr.q, base.q[:, perm]) and np.array_equal(pr.fidx, base.fidx)
    # the chosen error never exceeds plain round-to-nearest at f = 1.00
    assert np.all(base.mse[np.arange(5), base.fidx] <= base.mse[:, 30])
    # an all-zero row: scale 0, codes 0, index 0; -128 is reachable
    z = r.copy(); z[3] = 0
    zr = O.quantize_residual_w8(z)
    assert zr.fidx[3] == 0 and zr.scale[3] == 0 and np.all(zr.q[3] == 0)
    neg = np.linspace(-1.0, 0.4, 256)[None, :]
    assert O.quantize_residual_w8(neg).q.min() == -128
    assert base.q.min() >= -128 and base.q.max() <= 127


def pin_w8_layer():
    rng = np.random.default_rng(24)
    n, k, rank = 48, 512, 16
    w = rng.standard_normal((n, k)) / np.sqrt(k)
    up, dn = O.svd_init(w, rank)
    res = O.quantize_weight_w8(w, up, dn)
    w_hat = O.reconstruct_w8(res.q, res.scale, up, dn)
    # the weight round-trips within the int8 grid's error (a step of about
    # 3.3 sigma / 127 per row), well inside the W4 mode's
    assert O.rel_fro(w_hat, w) < 1e-2
    w4 = O.quantize_weight(w, *O.svd_init(w, 32), 32)
    assert O.rel_fro(w_hat, w) < O.rel_fro(O.reconstruct(w4.q, w4.scale, *O.svd_init(w, 32), 32), w)
    x = rng.standard_normal((7, k))
    y = O.forward_w8(x, res.q, res.scale, up, dn)
    assert np.allclose(y, x @ w_hat.T, rtol=1e-12, atol=1e-12)            # y = x W_hat^T
    d = O.forward_w8_fp16_operands(x, res.q, res.scale, up, dn)
    assert O.rel_fro(d, y) < 1e-3
    # rank 0: the residual is the rotated weight itself
    r0 = O.quantize_weight_w8(w, np.zeros((n, 0)), np.zeros((k, 0)))
    assert np.array_equal(r0.q, O.quantize_residual_w8(O.rotate(w)).q)


def pin_w8_certification():
    rng = np.random.default_rng(25)
    r = rng.standard_normal((40, 768)) * 0.01
    res = O.quantize_residual_w8(r)
    rep = O.check_device_quant_w8(r, res, res.q, res.scale, res.fidx)
    assert rep["ok"] and rep["differ"] == 0
    rows, near = O.certify_w8(r, res)
    assert rows.mean() > 0.8
    i = int(np.argwhere(rows)[0][0])
    j = int(np.argwhere(~near[i])[0][0])
    qd = res.q.copy()
    qd[i, j] = qd[i, j] + 1 if qd[i, j] < 127 else 126                   # one wrong code
    assert not O.check_device_quant_w8(r, res, qd, res.scale, res.fidx)["ok"]
    fd = res.fidx.copy(); fd[i] = (fd[i] + 7) % 31                          # a consistent wrong index
    sd = res.scale.copy(); sd[i] = O.fp16_round(O.candidate_scale_exact_w8(res.absmax[i], fd[i]))
    qd = res.q.copy(); qd[i] = O.codes_for_scale_w8(r[i], sd[i])
    assert not O.check_device_quant_w8(r, res, qd, sd, fd)["ok"]


# ----------------------------------------------------------------- MXFP4 mode
# E2M1 code points as the OCP Microscaling Formats v1.0 specification lists
# them (FP4 E2M1: +-0, 0.5, 1, 1.5, 2, 3, 4, 6), by nibble s e1 e0 m.
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def pin_mx_e2m1_table():
    v = O.e2m1_values()
    assert list(v[:8]) == OCP_E2M1
    assert list(-v[8:]) == OCP_E2M1
    # every code decodes and re-encodes to itself; -0 encodes as +0
    codes = np.arange(16, dtype=np.uint8)
    back = O.e2m1_encode(v)
    assert np.array_equal(back[codes != 8], codes[codes != 8]) and back[8] == 0


def pin_mx_encode_nearest_and_ties():
    rng = np.random.default_rng(40)
    v = np.concatenate([rng.uniform(-8, 8, 4000), rng.uniform(-0.6, 0.6, 1000)])
    c = O.e2m1_encode(v)
    dq = O.e2m1_values()[c]
    grid = np.array(OCP_E2M1 + [-g for g in OCP_E2M1[1:]])
    target = np.clip(v, -6, 6)                       # saturation
    best = np.abs(target[:, None] - grid[None, :]).min(axis=1)
    assert np.all(np.abs(target - dq) <= best + 1e-15)
    # midpoints go to the even mantissa: 0.25->0, 0.75->1, 1.25->1, 1.75->2,
    # 2.5->2, 3.5->4, 5->4; the sign follows
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    assert np.array_equal(O.e2m1_values()[O.e2m1_encode(ties)], want)
    assert np.array_equal(O.e2m1_values()[O.e2m1_encode(-ties)], -want)
    assert O.e2m1_encode(np.array([-0.2]))[0] == 0    # rounds to zero: nibble 0


def pin_mx_scale_rule():
    rng = np.random.default_rng(41)
    for p in (-20, -3, 0, 1, 5, 30):
        blk = rng.uniform(-1, 1, (1, 32)) * 2.0 ** p
        blk[0, 7] = 2.0 ** p                          # absmax exactly 2^p
        c, e = O.mx_quantize(blk)
        assert int(e[0, 0]) == p - 2 + 127
        assert O.e2m1_values()[c[0, 7]] == 4.0        # 2^p / 2^(p-2)
        blk[0, 7] = 6 * 2.0 ** p                      # 6 x 2^p is on the grid at e = p + 127
        c, e = O.mx_quantize(blk)
        assert int(e[0, 0]) == p + 127 and c[0, 7] == 7
        # scaling the block by 2^k moves the exponent by k and keeps the nibbles
        c2, e2 = O.mx_quantize(blk * 2.0 ** 9)
        assert np.array_equal(c2, c) and int(e2[0, 0]) == int(e[0, 0]) + 9
    c, e = O.mx_quantize(np.zeros((1, 32)))
    assert e[0, 0] == 0 and not c.any()
    c, e = O.mx_quantize(np.full((1, 32), 2.0 ** -140))
    assert e[0, 0] == 0                               # clamped at the smallest scale


def pin_mx_error_bound():
    rng = np.random.default_rng(42)
    a = rng.standard_normal((16, 256)) * np.exp(rng.standard_normal((16, 1)))
    c, e = O.mx_quantize(a)
    err = np.abs(O.mx_dequant(c, e) - a)
    x = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)
    # half the largest grid spacing (4 -> 6) up to 6X; saturation above (< 8X)
    assert np.all(np.where(np.abs(a) <= 6 * x, err <= x, err <= 2 * x))
    # and the block maximum (in [4X, 8X)) keeps its sign and lands on 4 or 6
    blocks = a.reshape(16, 8, 32)
    i = np.abs(blocks).argmax(axis=-1)
    top = np.take_along_axis(c.reshape(16, 8, 32), i[..., None], -1)[..., 0]
    assert set(np.unique(top & 7)) <= {6, 7}


def pin_mx_pack():
    c = np.array([[1, 2, 15, 8, 0, 7]], dtype=np.uint8)
    p = O.mx_pack(c)
    assert list(p[0]) == [0x21, 0x8F, 0x70]
    assert np.array_equal(O.mx_unpack(p), c)


def pin_mx_forward_on_grid():
    # activations whose rotation is exactly representable: the FP4 forward is
    # then x @ W_hat^T with W_hat the MXFP4 reconstruct, to fp64 rounding
    rng = np.random.default_rng(43)
    m, n, k, r = 5, 24, 512, 4
    grid = np.array(OCP_E2M1 + [-g for g in OCP_E2M1[1:]])
    xh = grid[rng.integers(0, 15, (m, k))] * np.repeat(2.0 ** rng.integers(-6, 4, (m, k // 32)), 32, axis=1)
    x = O.rotate(xh)
    w = rng.standard_normal((n, k)) * 0.05
    up = O.bf16_round(rng.standard_normal((n, r)) * 0.1)
    dn = O.bf16_round(rng.standard_normal((k, r)) * 0.1)
    wc, we = O.quantize_weight_mx(w, up, dn)
    y = O.forward_mx(x, wc, we, up, dn)
    ref = x @ O.reconstruct_mx(wc, we, up, dn).T
    assert O.rel_fro(y, ref) < 1e-12
    # the weight side alone: reconstruct recovers W up to the FP4 error of R
    wh = O.reconstruct_mx(wc, we, up, dn)
    e = O.residual(w, up, dn)
    assert O.rel_fro(wh, w) <= 0.2 * np.linalg.norm(e) / np.linalg.norm(w) + 1e-12


def pin_mx_layer():
    from synth import gen_weight, gen_activations, bf16_bits_to_f32
    rng = np.random.default_rng(44)
    w = gen_weight(rng, 96, 512, 4).astype(np.float64)
    x = bf16_bits_to_f32(gen_activations(rng, 16, 512, 0.01)).astype(np.float64)
    up, dn = O.svd_init(w, 32)
    wc, we = O.quantize_weight_mx(w, up, dn)
    wh = O.reconstruct_mx(wc, we, up, dn)
    res4 = O.quantize_residual(O.residual(w, up, dn), 32)
    wh4 = O.reconstruct(res4.q, res4.scale, up, dn, 32)
    e_mx, e_4 = O.rel_fro(wh, w), O.rel_fro(wh4, w)
    assert e_4 < e_mx < 0.1          # the swept int4 grid beats the plain FP4 one
    y = O.forward_mx(x, wc, we, up, dn)
    assert O.cosine(y, x @ w.T) > 0.99


def pin_mx_certification():
    rng = np.random.default_rng(45)
    a = rng.standard_normal((32, 256))
    c, e = O.mx_quantize(a)
    rep = O.check_device_mx(a, c, e)
    assert rep["ok"] and rep["differ"] == 0
    ok, near = O.certify_mx(a, e)
    i, j = np.argwhere(~near)[0]
    c2 = c.copy(); c2[i, j] = (c2[i, j] + 1) & 15 if (c2[i, j] & 7) < 7 else c2[i, j] - 1
    assert not O.check_device_mx(a, c2, e)["ok"]
    e2 = e.copy(); e2[i, j // 32] += 1
    c3, _ = O.mx_quantize(a)
    assert not O.check_device_mx(a, c3, e2)["ok"]


# ----------------------------------------------------------------- metrics and decoders
def pin_metrics_closed_forms():
    # rel_F(a, b) = ||a - b|| / ||b||: normalised by the second argument
    b = np.array([3.0, 4.0])                          # ||b|| = 5
    a = np.array([3.0, 5.0])                          # ||a - b|| = 1, ||a|| = sqrt(34)
    assert O.rel_fro(a, b) == 0.2
    assert abs(O.rel_fro(b, a) - 1 / np.sqrt(34)) < 1e-15
    assert O.rel_fro(b, b) == 0.0
    assert O.rel_fro(2 * b, b) == 1.0 and O.rel_fro(-b, b) == 2.0
    # the Frobenius norm of a matrix is that of its flattened entries
    m = np.array([[1.0, 2.0], [2.0, 4.0]])            # ||m||_F = 5
    assert O.rel_fro(m + np.array([[0.0, 0.0], [0.0, 3.0]]), m) == 0.6
    # cos = <a, b> / (||a|| ||b||): scale-free, signed
    assert O.cosine([1.0, 0.0], [0.0, 7.0]) == 0.0
    assert abs(O.cosine([2.0, 0.0], [1.0, 1.0]) - 1 / np.sqrt(2)) < 1e-15
    assert abs(O.cosine(3 * b, b) - 1.0) < 1e-15 and abs(O.cosine(-b, 0.5 * b) + 1.0) < 1e-15
    assert abs(O.cosine(m, m.T) - 1.0) < 1e-15       # symmetric: same flattened vector
    assert abs(O.cosine([[1.0, 2.0], [3.0, 4.0]], [[1.0, 3.0], [2.0, 4.0]]) - 29 / 30) < 1e-15


def _fp16_by_formula(bits):
    """IEEE binary16 value of each 16-bit pattern: sign, 5-bit biased exponent, 10-bit fraction."""
    bits = np.asarray(bits, np.int64)
    sgn = np.where(bits >> 15, -1.0, 1.0)
    e = (bits >> 10) & 31
    f = (bits & 1023).astype(np.float64)
    v = np.where(e == 0, f * 2.0 ** -24, (1 + f / 1024) * np.ldexp(1.0, (e - 15).astype(np.int64)))
    v = np.where(e == 31, np.where(f == 0, np.inf, np.nan), v)
    return sgn * v


def _bf16_by_formula(bits):
    """bfloat16 value of each 16-bit pattern: sign, 8-bit biased exponent, 7-bit fraction."""
    bits = np.asarray(bits, np.int64)
    sgn = np.where(bits >> 15, -1.0, 1.0)
    e = (bits >> 7) & 255
    f = (bits & 127).astype(np.float64)
    v = np.where(e == 0, f * 2.0 ** -133, (1 + f / 128) * np.ldexp(1.0, (e - 127).astype(np.int64)))
    v = np.where(e == 255, np.where(f == 0, np.inf, np.nan), v)
    return sgn * v


def pin_fp16_bf16_decode_all_patterns():
    allbits = np.arange(65536).astype(np.uint16)
    assert np.array_equal(O.fp16_decode(allbits), _fp16_by_formula(allbits), equal_nan=True)
    assert np.array_equal(O.bf16_decode(allbits), _bf16_by_formula(allbits), equal_nan=True)
    # an fp16 array decodes to its own values
    h = np.array([0.5, -3.25, 65504.0, 2.0 ** -24], np.float16)
    assert list(O.fp16_decode(h)) == [0.5, -3.25, 65504.0, 2.0 ** -24]


def pin_w8_fp16_operand_forward():
    rng = np.random.default_rng(26)
    n, k, m = 20, 512, 6
    q = rng.integers(-128, 128, (n, k)).astype(np.float64)
    sc = O.fp16_round(rng.uniform(1e-3, 1e-2, n))
    up = O.bf16_round(rng.standard_normal((n, 16)) * 0.1)
    dn = O.bf16_round(rng.standard_normal((k, 16)) * 0.1)
    # activations whose rotation is fp16-exact after the row power of two:
    # then the diagnostic forward equals the exact one
    xi = O.rotate(rng.integers(-40, 41, (m, k)).astype(np.float64) / 4)
    np.testing.assert_allclose(O.forward_w8_fp16_operands(xi, q, sc, up, dn),
                               O.forward_w8(xi, q, sc, up, dn), rtol=1e-12, atol=1e-12)
    # in general only the rotated activations round (relative 2^-11 each)
    x = O.bf16_round(rng.standard_normal((m, k)) * 5)
    y = O.forward_w8(x, q, sc, up, dn)
    yd = O.forward_w8_fp16_operands(x, q, sc, up, dn)
    xh = O.rotate(x)
    bound = (np.abs(xh) @ np.abs(q).T) * np.abs(sc)[None, :] * 2.0 ** -11
    assert np.all(np.abs(yd - y) <= bound * (1 + 1e-9))
    e = O.rel_fro(yd, y)
    assert 1e-6 < e < 2.0 ** -11


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------- planted mistakes
def _mutations():
    """Plausible mistakes, each planted in the oracle on the CPU."""
    orig_h = O.sq_oracle.hadamard256
    orig_codes = O.sq_oracle.codes_for_scale
    orig_dequant = O.sq_oracle.dequant
    orig_fwd = O.sq_oracle.forward
    orig_pack = O.sq_oracle.pack
    orig_scale = O.sq_oracle.candidate_scale_exact
    orig_svd = O.sq_oracle.svd_init

    def unnormalised():
        return orig_h() * 16

    def half_away(r, s):
        r = np.asarray(r, float); s = np.asarray(s, float)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = r / s
            q = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -8, 7)
        return np.where(s == 0, 0.0, q)

    def symmetric_clamp(r, s):
        return np.clip(orig_codes(r, s), -7, 7)

    def tiled_groups(q, scale, group):
        q = np.asarray(q, float)
        return q * np.tile(np.asarray(scale, float), group)

    def dropped_lowrank(x, q, scale, up, down, group):
        return orig_fwd(x, q, scale, up[:, :0], down[:, :0], group)

    def dgrad_unrotated(dy, q, scale, up, down, group):
        dy = np.asarray(dy, float)
        return dy @ orig_dequant(q, scale, group) + (dy @ up) @ down.T

    def dgrad_swapped_factors(dy, q, scale, up, down, group):
        dy = np.asarray(dy, float)
        return O.rotate(dy @ orig_dequant(q, scale, group)) + (dy @ up[:, ::-1]) @ down.T

    def swapped_nibbles(q):
        q = np.asarray(q).astype(np.int64)
        return ((q[..., 1::2] & 0xF) | ((q[..., 0::2] & 0xF) << 4)).astype(np.uint8)

    def fraction_off_by_one(a, i):
        return orig_scale(a, np.asarray(i) + 1)

    orig_codes8 = O.sq_oracle.codes_for_scale_w8
    orig_scale8 = O.sq_oracle.candidate_scale_exact_w8

    def symmetric_clamp_w8(r, s):
        return np.clip(orig_codes8(r, s), -127, 127)

    def w8_divisor_7(a, i):
        return orig_scale8(a, i) * 127 / 7

    def w8_scale_per_column(q, scale):
        q = np.asarray(q, float)
        return q * np.resize(np.asarray(scale, float), q.shape[1])[None, :]

    def svd_no_sqrt(w, rank=32, round_bf16=True):
        w = np.asarray(w, float)
        u, s, vt = np.linalg.svd(w, full_matrices=False)
        up, dn = u[:, :rank] * s[:rank], vt[:rank].T * s[:rank]
        return (O.bf16_round(up), O.bf16_round(dn)) if round_bf16 else (up, dn)

    orig_enc = O.sq_oracle.e2m1_encode
    orig_mxe = O.sq_oracle.mx_scale_exponent
    orig_mxdq = O.sq_oracle.mx_dequant

    def e2m1_ties_away(v):
        v = np.asarray(v, float)
        c = orig_enc(v)
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        up_one = np.isin(np.abs(v), mids)
        bumped = np.where(up_one & ((c & 7) < 7), c + 1, c)
        return np.where(up_one & (v < 0) & ((c & 7) == 0), 9, bumped).astype(np.uint8)

    def mx_scale_ceil(a):
        a = np.asarray(a, float)
        e = orig_mxe(a).astype(np.int64)
        with np.errstate(divide="ignore"):
            frac = np.log2(np.where(a > 0, a, 1.0)) % 1 != 0
        return np.clip(e + frac, 0, 254).astype(np.uint8)

    def mx_scale_emax3(a):
        return np.clip(orig_mxe(a).astype(np.int64) - 1, 0, 254).astype(np.uint8)

    def mx_dequant_tiled(codes, exps):
        codes = np.asarray(codes, np.uint8)
        v = O.e2m1_values()[codes]
        s = np.ldexp(1.0, np.asarray(exps).astype(np.int64) - 127)
        return v * np.tile(s, (1, 32))

    def act_unrotated(x):
        return O.mx_quantize(np.asarray(x, float))

    def rel_fro_by_a(a, b):
        a = np.asarray(a, float).ravel(); b = np.asarray(b, float).ravel()
        return float(np.linalg.norm(a - b) / np.linalg.norm(a))

    def rel_fro_squared(a, b):
        a = np.asarray(a, float).ravel(); b = np.asarray(b, float).ravel()
        return float((np.linalg.norm(a - b) / np.linalg.norm(b)) ** 2)

    def cosine_one_norm(a, b):
        a = np.asarray(a, float).ravel(); b = np.asarray(b, float).ravel()
        return float(a @ b / np.linalg.norm(b) ** 2)

    def fp16_decode_as_int(h):
        return np.asarray(h).astype(np.float64)

    def bf16_decode_low_half(bits):
        b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
        return b.view(np.float32).astype(np.float64)

    orig_fwd8d = O.sq_oracle.forward_w8_fp16_operands

    def fwd8_scale_twice(x, q, scale, up, down):
        y = orig_fwd8d(x, q, scale, up, down)
        lr = (np.asarray(x, float) @ down) @ up.T
        return (y - lr) * np.asarray(scale, float)[None, :] + lr

    def fwd8_bf16_operands(x, q, scale, up, down):
        x = np.asarray(x, float)
        xh = O.bf16_round(O.rotate(x))
        return (xh @ np.asarray(q, float).T) * np.asarray(scale, float)[None, :] + (x @ down) @ up.T

    return [
        ("rel_fro", rel_fro_by_a),
        ("rel_fro", rel_fro_squared),
        ("cosine", cosine_one_norm),
        ("fp16_decode", fp16_decode_as_int),
        ("bf16_decode", bf16_decode_low_half),
        ("forward_w8_fp16_operands", fwd8_scale_twice),
        ("forward_w8_fp16_operands", fwd8_bf16_operands),
        ("e2m1_encode", e2m1_ties_away),
        ("mx_scale_exponent", mx_scale_ceil),
        ("mx_scale_exponent", mx_scale_emax3),
        ("mx_dequant", mx_dequant_tiled),
        ("quantize_act_mx", act_unrotated),
        ("hadamard256", unnormalised),
        ("codes_for_scale", half_away),
        ("codes_for_scale", symmetric_clamp),
        ("dequant", tiled_groups),
        ("forward", dropped_lowrank),
        ("dgrad", dgrad_unrotated),
        ("dgrad", dgrad_swapped_factors),
        ("pack", swapped_nibbles),
        ("candidate_scale_exact", fraction_off_by_one),
        ("svd_init", svd_no_sqrt),
        ("codes_for_scale_w8", symmetric_clamp_w8),
        ("candidate_scale_exact_w8", w8_divisor_7),
        ("dequant_w8", w8_scale_per_column),
    ]


@pytest.mark.parametrize("name,mutant", _mutations(), ids=lambda v: getattr(v, "__name__", str(v)))
def test_planted_mistakes(monkeypatch, name, mutant):
    monkeypatch.setattr(O.sq_oracle, name, mutant)
    monkeypatch.setattr(O, name, mutant, raising=False)
    if name == "hadamard256":
        monkeypatch.setattr(O.sq_oracle, "_H", None)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake in {name}"
