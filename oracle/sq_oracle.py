"""Plain CPU fp64 oracle for the SquareQ v3 W4 linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the device library and never imports it.

Source: the SquareQ README (github.itlym.cn/CodeAlexx/SquareQ), section
"SquareQ v3 - W4 (Hadamard-256 + low-rank + int4 / NVFP4)":

* the weight is the sum of a bf16 low-rank product lora_up @ lora_down^T
  and the inverse block Hadamard-256 rotation of a dequantized residual
  (the format formula at the top of the section);
* the rotation is a block-diagonal normalized Hadamard-256 over the input
  dimension, for any K divisible by 256 (the "Rotation" bullet);
* the residual codec is int4 with group-32 or group-64 scales whose
  fraction is chosen by an MSE sweep (the "Residual codecs" bullet; the
  sweep grid f in {0.70, 0.71, ..., 1.00} with scale f*absmax/7 and codes
  in [-8, 7] is the one the layer configurations state);
* the low-rank branch is a rank-32 SVD of the weight, stored in bf16 (the
  "Low-rank branch" bullet);
* the selftest gates named in the "Layout" paragraph (pack/unpack
  bit-exact, rotation self-inverse, determinism) are among the pins.

Everything is numpy float64; LAPACK SVD and BLAS matmul are the only
library primitives.  Points the page leaves open are decided as follows
(each decision is repeated where it is used):

  R1 Hadamard order: Sylvester, S[i,j] = (-1)^popcount(i & j); H = S/16.
  R2 side: each row is rotated along K; R = E @ H (H symmetric, H @ H = I).
  R3 SVD split: up = U*sqrt(S), down = V*sqrt(S), rounded to bf16 straight
     from fp64; the residual is taken against the rounded factors.
  R4 scales are stored as IEEE fp16; each candidate scale is rounded to
     fp16 before its codes and error are computed.
  R5 codes: round half to even, clamp to [-8, 7]; a zero scale gives code 0.
  R6 the sweep minimises the sum of squared errors in the rotated domain;
     ties go to the lowest fraction index.
  R7 packing: byte b = (q[2b] & 0xF) | (q[2b+1] & 0xF) << 4, two's complement.

The int8-residual mode (the page's "v3.1 - int8-residual mode" section) is at
the end of the module, with its own readings W1-W5.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HBLOCK = 256
N_FRAC = 31          # f = 0.70 ... 1.00 in steps of 0.01
QMIN, QMAX = -8, 7


# --------------------------------------------------------------------------
# floating-point formats (written from the IEEE definitions)
# --------------------------------------------------------------------------
def _round_to_format(x, sig_bits: int, emin: int, max_finite: float) -> np.ndarray:
    """Round fp64 values to a binary format with ``sig_bits`` significant bits.

    Round to nearest, ties to even, with gradual underflow below 2**emin and
    overflow to +-inf when the rounded magnitude exceeds ``max_finite``.
    One rounding straight from fp64 (no intermediate format).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, emin + 1)                  # subnormal range: fixed spacing
    spacing = np.ldexp(1.0, e - sig_bits)
    r = np.rint(x[fin] / spacing) * spacing      # division by a power of two: exact
    r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, r), r)
    out[fin] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def fp16_round(x) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of fp64 values (returned as fp64)."""
    return _round_to_format(x, 11, -14, 65504.0)


def bf16_round(x) -> np.ndarray:
    """bfloat16 round-to-nearest-even of fp64 values (returned as fp64)."""
    return _round_to_format(x, 8, -126, float.fromhex("0x1.fep127"))


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_decode(h) -> np.ndarray:
    """fp16 array or uint16 bit patterns -> fp64 values."""
    h = np.asarray(h)
    if h.dtype == np.uint16:
        h = h.view(np.float16)
    return h.astype(np.float64)


# --------------------------------------------------------------------------
# Hadamard-256 (the "Rotation" bullet; readings R1, R2)
# --------------------------------------------------------------------------
def sylvester(n: int = HBLOCK) -> np.ndarray:
    """S[i,j] = (-1)^popcount(i & j), the natural-order Sylvester matrix."""
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


_H = None


def hadamard256() -> np.ndarray:
    """Normalized Hadamard-256: H = S/16, symmetric and its own inverse."""
    global _H
    if _H is None:
        _H = sylvester(HBLOCK) / 16.0
    return _H


def rotate(a) -> np.ndarray:
    """Apply the block-diagonal H to every row: out[:, 256b:256b+256] = a[:, block b] @ H.

    K must be a multiple of 256.  The same map is its own inverse.
    """
    a = np.asarray(a, dtype=np.float64)
    k = a.shape[-1]
    if k % HBLOCK:
        raise ValueError("K must be a multiple of 256")
    blocks = a.reshape(a.shape[:-1] + (k // HBLOCK, HBLOCK))
    return (blocks @ hadamard256()).reshape(a.shape)


def fwht_fast(a) -> np.ndarray:
    """The same rotation through radix-2 butterflies (a+b, a-b), then x 1/16.

    Independent of the dense matrix above; used to cross-check it.
    """
    a = np.array(a, dtype=np.float64, copy=True)
    k = a.shape[-1]
    v = a.reshape(-1, k // HBLOCK, HBLOCK)
    h = 1
    while h < HBLOCK:
        v = v.reshape(v.shape[0], v.shape[1], HBLOCK // (2 * h), 2, h)
        lo = v[:, :, :, 0, :].copy()
        hi = v[:, :, :, 1, :].copy()
        v[:, :, :, 0, :] = lo + hi
        v[:, :, :, 1, :] = lo - hi
        h *= 2
    return (v.reshape(a.shape) / 16.0)


# --------------------------------------------------------------------------
# low-rank branch (the "Low-rank branch" bullet; reading R3)
# --------------------------------------------------------------------------
def svd_init(w, rank: int = 32, round_bf16: bool = True):
    """Rank-``rank`` split of W: up = U_r sqrt(S_r), down = V_r sqrt(S_r), bf16-rounded.

    Returns (up [N,r], down [K,r]) as fp64 arrays holding bf16 values
    (unrounded when ``round_bf16`` is False, for the Eckart-Young pin).
    Only the product up @ down^T is meaningful (signs of singular vectors
    are arbitrary).
    """
    w = np.asarray(w, dtype=np.float64)
    if rank == 0:
        return np.zeros((w.shape[0], 0)), np.zeros((w.shape[1], 0))
    u, s, vt = np.linalg.svd(w, full_matrices=False)
    r = np.sqrt(s[:rank])
    up = u[:, :rank] * r
    down = vt[:rank].T * r
    if round_bf16:
        up, down = bf16_round(up), bf16_round(down)
    return up, down


def residual(w, up, down) -> np.ndarray:
    """Rotated residual R = rotate(W - up @ down^T) (format formula, reading R2)."""
    w = np.asarray(w, dtype=np.float64)
    e = w - np.asarray(up, np.float64) @ np.asarray(down, np.float64).T
    return rotate(e)


# --------------------------------------------------------------------------
# int4 codec with MSE-swept fractional scales (the "Residual codecs" bullet)
# --------------------------------------------------------------------------
def fractions_grid() -> np.ndarray:
    """The 31 candidate fractions f_i = (70 + i)/100."""
    return (70 + np.arange(N_FRAC)) / 100.0


def candidate_scale_exact(absmax, i):
    """Unrounded candidate scale f_i * absmax / 7 = (70+i)*absmax/700 (fp64)."""
    return (70.0 + i) * np.asarray(absmax, np.float64) / 700.0


def codes_for_scale(r, s) -> np.ndarray:
    """Reading R5: q = clamp(round_half_even(r/s), -8, 7); q = 0 where s == 0."""
    r = np.asarray(r, np.float64)
    s = np.asarray(s, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(r / s), QMIN, QMAX)
    return np.where(s == 0, 0.0, q)


@dataclass
class QuantResult:
    q: np.ndarray        # int codes [N,K] (int8)
    scale: np.ndarray    # fp16 scale values [N,K/G] (float64 holding fp16 values)
    fidx: np.ndarray     # chosen fraction index [N,K/G] (uint8)
    mse: np.ndarray      # [N,K/G,31] sum of squared errors per candidate
    absmax: np.ndarray   # [N,K/G]


def quantize_residual(r, group: int) -> QuantResult:
    """Sweep the 31 fractions for every group of ``group`` values along K.

    For group values r_1..r_G with absmax a, candidate i uses
    s_i = fp16(f_i a / 7) (reading R4), codes q = clamp(rint(r/s_i), -8, 7)
    (R5) and error sum (r - q s_i)^2; the chosen index is the first
    minimiser (R6).  Non-finite inputs or an fp16 scale overflow raise.
    """
    r = np.asarray(r, np.float64)
    n, k = r.shape
    if group not in (32, 64) or k % HBLOCK:
        raise ValueError("group must be 32 or 64 and K a multiple of 256")
    if not np.all(np.isfinite(r)):
        raise FloatingPointError("non-finite residual")
    rg = r.reshape(n, k // group, group)
    a = np.abs(rg).max(axis=2)
    mse = np.empty((n, k // group, N_FRAC))
    scales = np.empty((n, k // group, N_FRAC))
    for i in range(N_FRAC):
        s = fp16_round(candidate_scale_exact(a, i))
        if np.any(np.isinf(s)):
            raise FloatingPointError("fp16 scale overflow")
        q = codes_for_scale(rg, s[..., None])
        mse[..., i] = ((rg - q * s[..., None]) ** 2).sum(axis=2)
        scales[..., i] = s
    best = np.argmin(mse, axis=2)          # numpy argmin returns the first minimum
    s_best = np.take_along_axis(scales, best[..., None], axis=2)[..., 0]
    q_best = codes_for_scale(rg, s_best[..., None]).reshape(n, k)
    return QuantResult(q_best.astype(np.int8), s_best, best.astype(np.uint8), mse, a)


def quantize_weight(w, up, down, group: int) -> QuantResult:
    """Builder path: residual against the bf16 factors, rotation, sweep."""
    return quantize_residual(residual(w, up, down), group)


def pack(q) -> np.ndarray:
    """Reading R7: two's-complement nibbles, even k in the low nibble."""
    q = np.asarray(q).astype(np.int64)
    if q.shape[-1] % 2:
        raise ValueError("even K required")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack(codes) -> np.ndarray:
    """Inverse of ``pack``: uint8 [N,K/2] -> int8 [N,K] in [-8, 7]."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    lo = c & 0xF
    hi = c >> 4
    q = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    q = np.where(q >= 8, q - 16, q)
    return q.astype(np.int8)


def dequant(q, scale, group: int) -> np.ndarray:
    """D = q * s with s repeated over each group (exact in fp64)."""
    q = np.asarray(q, np.float64)
    s = np.repeat(np.asarray(scale, np.float64), group, axis=-1)
    return q * s


# --------------------------------------------------------------------------
# the layer (format formula)
# --------------------------------------------------------------------------
def reconstruct(q, scale, up, down, group: int) -> np.ndarray:
    """W_hat = up @ down^T + rotate(dequant(R)) in fp64 (format formula)."""
    lr = np.asarray(up, np.float64) @ np.asarray(down, np.float64).T
    return lr + rotate(dequant(q, scale, group))


def forward(x, q, scale, up, down, group: int) -> np.ndarray:
    """y = x @ W_hat^T = rotate(x) @ D^T + (x @ down) @ up^T in fp64.

    The two halves follow from the format formula: H is symmetric, so
    x @ (D H)^T = (x H) @ D^T.
    """
    x = np.asarray(x, np.float64)
    d = dequant(q, scale, group)
    return rotate(x) @ d.T + (x @ np.asarray(down, np.float64)) @ np.asarray(up, np.float64).T


def forward_fp16_operands(x, q, scale, up, down, group: int) -> np.ndarray:
    """Diagnostic forward: the contraction's operands rounded to fp16.

    The rotated activations of each row are multiplied by the power of two
    2^(11-E), E = ceil(log2(max|x_row|)) (so every |x H| <= 16 max|x| maps
    below 2^15), rounded to fp16, and the dequantized weight is rounded to
    fp16 (q*s rounded once); the row factor is undone afterwards and the
    low-rank term is exact.  A device contraction on fp16 operands with fp32
    accumulation should agree with this to accumulation-order error.
    """
    x = np.asarray(x, np.float64)
    xh = rotate(x)
    amax = np.abs(x).max(axis=1)
    e = np.zeros(x.shape[0])
    nz = amax > 0
    # smallest E with amax <= 2**E
    mant, ex = np.frexp(amax[nz])
    e[nz] = np.where(mant == 0.5, ex - 1, ex)
    f = np.ldexp(1.0, (11 - e).astype(np.int64))
    xh16 = fp16_round(xh * f[:, None])
    d16 = fp16_round(dequant(q, scale, group))
    y = (xh16 @ d16.T) / f[:, None]
    return y + (x @ np.asarray(down, np.float64)) @ np.asarray(up, np.float64).T


def dgrad(dy, q, scale, up, down, group: int) -> np.ndarray:
    """Input gradient of the layer: dx = dy @ W_hat in fp64.

    From the format formula, dy @ (up @ down^T + D H) = (dy @ D) H +
    (dy @ up) @ down^T with D = dequant(R): the int4 product contracts over
    the output features and the rotation acts on its result's K blocks.
    """
    dy = np.asarray(dy, np.float64)
    d = dequant(q, scale, group)
    return rotate(dy @ d) + (dy @ np.asarray(up, np.float64)) @ np.asarray(down, np.float64).T


def dgrad_fp16_operands(dy, q, scale, up, down, group: int) -> np.ndarray:
    """Diagnostic input gradient: the int4 contraction's operands in fp16.

    Each row of dy is multiplied by 2^(11-E), E = ceil(log2(max|dy_row|)),
    and rounded to fp16; the dequantized weight is fp16(q*s); the product is
    rotated, the row factor undone, and the low-rank term is exact.
    """
    dy = np.asarray(dy, np.float64)
    amax = np.abs(dy).max(axis=1)
    e = np.zeros(dy.shape[0])
    nz = amax > 0
    mant, ex = np.frexp(amax[nz])
    e[nz] = np.where(mant == 0.5, ex - 1, ex)
    f = np.ldexp(1.0, (11 - e).astype(np.int64))
    dy16 = fp16_round(dy * f[:, None])
    d16 = fp16_round(dequant(q, scale, group))
    dx = rotate(dy16 @ d16) / f[:, None]
    return dx + (dy @ np.asarray(up, np.float64)) @ np.asarray(down, np.float64).T


# --------------------------------------------------------------------------
# metrics
# --------------------------------------------------------------------------
def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F over the flattened arrays, fp64."""
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb else float(np.linalg.norm(a))


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# --------------------------------------------------------------------------
# tie certification for comparing a fp32 device quantizer with this oracle
# --------------------------------------------------------------------------
SCALE_MARGIN = 1e-5   # relative distance of f*a/7 from an fp16 rounding boundary
CODE_MARGIN = 2e-4    # distance of r/s from a half-integer, in code units
SWEEP_MARGIN = 1e-4   # relative gap between best and any other candidate


def _fp16_bracket(v):
    """(lo, hi): the fp16 values with lo <= v <= hi that are adjacent (v >= 0)."""
    v = np.asarray(v, np.float64)
    s = fp16_round(v).astype(np.float16)
    up = np.nextafter(s, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(s, np.float16(0)).astype(np.float64)
    s = s.astype(np.float64)
    lo = np.where(s <= v, s, dn)
    hi = np.where(s >= v, s, up)
    return lo, hi


def _fp16_boundary_margin(v) -> np.ndarray:
    """Relative distance of v (>= 0) from the nearest fp16 rounding boundary.

    The boundaries around v are the midpoints between the fp16 value that
    v rounds to and its two neighbours.
    """
    v = np.asarray(v, np.float64)
    s16 = fp16_round(v).astype(np.float16)
    s = s16.astype(np.float64)
    up = np.nextafter(s16, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(s16, np.float16(0)).astype(np.float64)
    d = np.minimum(np.abs(v - (s + up) / 2), np.abs(v - (s + dn) / 2))
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(v > 0, d / np.where(v > 0, v, 1), np.inf)
    return out


def _variant_mse(rg, a):
    """Error of every candidate under each admissible fp16 rounding of its scale.

    Returns (scales [.., 31, 2], mse [.., 31, 2]): variant 0 is the correct
    rounding; variant 1 is the other fp16 neighbour when the unrounded scale
    lies within SCALE_MARGIN of a rounding boundary, else a copy of variant 0.
    A device that computes the absmax in fp32 may take either variant there.
    """
    shape = a.shape + (N_FRAC, 2)
    sc = np.empty(shape)
    ms = np.empty(shape)
    for i in range(N_FRAC):
        v = candidate_scale_exact(a, i)
        s0 = fp16_round(v)
        lo, hi = _fp16_bracket(v)
        amb = _fp16_boundary_margin(v) <= SCALE_MARGIN
        s1 = np.where(amb, np.where(s0 == lo, hi, lo), s0)
        for j, sv in enumerate((s0, s1)):
            q = codes_for_scale(rg, sv[..., None])
            sc[..., i, j] = sv
            ms[..., i, j] = ((rg - q * sv[..., None]) ** 2).sum(axis=-1)
    return sc, ms


def certify(r, res: QuantResult, group: int):
    """Per-group flag: True where the oracle's choice is far from every tie.

    A group is certified when (a) the chosen unrounded scale is at least
    SCALE_MARGIN (relative) from an fp16 rounding boundary, (b) every r/s
    is at least CODE_MARGIN from a half-integer, and (c) every other
    candidate's error exceeds the best by SWEEP_MARGIN (relative), also when
    that candidate's scale would round the other way.  A device quantizer
    whose residual differs from the oracle's by fp32 rounding must then
    reproduce codes, scale and index bit for bit.
    """
    r = np.asarray(r, np.float64)
    n, k = r.shape
    rg = r.reshape(n, k // group, group)
    a = res.absmax
    best = res.fidx.astype(np.int64)
    ok = _fp16_boundary_margin(candidate_scale_exact(a, best)) > SCALE_MARGIN
    ok |= (a == 0)
    s = res.scale[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, rg / np.where(s > 0, s, 1), 0.0)
    frac = np.abs(t - np.floor(t) - 0.5)
    near = (frac < CODE_MARGIN) & (t > QMIN - 1) & (t < QMAX + 1)
    ok &= ~near.any(axis=2)
    _, ms = _variant_mse(rg, a)
    others = ms.min(axis=-1)
    np.put_along_axis(others, best[..., None], np.inf, axis=2)
    mse_best = np.take_along_axis(res.mse, best[..., None], axis=2)[..., 0]
    gap_ok = others.min(axis=2) > mse_best * (1 + SWEEP_MARGIN)
    gap_ok |= (a == 0)
    return ok & gap_ok


def check_device_quant(r, res: QuantResult, group: int, q_dev, scale_dev, fidx_dev):
    """Compare a device quantization with the oracle under tie certification.

    Returns a dict with counts; ``ok`` is True when certified groups match
    bit for bit and every other differing group is an admissible near-tie:
      * its scale is an admissible fp16 rounding of f_j a/7 for the device's
        index j (the correct one, or the other neighbour within SCALE_MARGIN);
      * its codes are the requantization with that scale, except values within
        CODE_MARGIN of a half-integer, which may take either neighbour;
      * its error is at most (1 + SWEEP_MARGIN) times the error of every other
        candidate i under the rounding of s_i least favourable to i, i.e. some
        admissible set of roundings makes the device's choice a minimiser.
    """
    r = np.asarray(r, np.float64)
    n, k = r.shape
    ng = k // group
    rg = r.reshape(n, ng, group)
    cert = certify(r, res, group)
    qd = np.asarray(q_dev).astype(np.int64).reshape(n, ng, group)
    qo = res.q.astype(np.int64).reshape(n, ng, group)
    sd = np.asarray(scale_dev, np.float64)
    fd = np.asarray(fidx_dev).astype(np.int64)
    same = (fd == res.fidx) & (sd == res.scale) & (qd == qo).all(axis=2)
    bad_cert = cert & ~same
    sc, ms = _variant_mse(rg, res.absmax)
    cand = np.take_along_axis(sc, np.clip(fd, 0, N_FRAC - 1)[..., None, None], axis=2)[..., 0, :]
    scale_ok = (sd == cand[..., 0]) | (sd == cand[..., 1])
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(sd[..., None] > 0, rg / np.where(sd[..., None] > 0, sd[..., None], 1), 0.0)
    q_req = np.clip(np.rint(t), QMIN, QMAX)
    near = np.abs(t - np.floor(t) - 0.5) < CODE_MARGIN
    q_lo = np.clip(np.floor(t), QMIN, QMAX)
    q_hi = np.clip(np.ceil(t), QMIN, QMAX)
    codes_ok = ((qd == q_req) | (near & ((qd == q_lo) | (qd == q_hi)))).all(axis=2)
    mse_dev = ((rg - qd * sd[..., None]) ** 2).sum(axis=2)
    worst = ms.max(axis=-1)
    np.put_along_axis(worst, np.clip(fd, 0, N_FRAC - 1)[..., None], np.inf, axis=2)
    err_ok = mse_dev <= worst.min(axis=2) * (1 + SWEEP_MARGIN)
    err_ok |= (res.absmax == 0) & (mse_dev == 0)
    admissible = scale_ok & codes_ok & err_ok & (fd >= 0) & (fd < N_FRAC)
    bad_uncert = ~cert & ~same & ~admissible
    return {
        "groups": int(n * ng),
        "uncertified": int((~cert).sum()),
        "differ": int((~same).sum()),
        "bad_certified": int(bad_cert.sum()),
        "bad_uncertified": int(bad_uncert.sum()),
        "ok": bool(bad_cert.sum() == 0 and bad_uncert.sum() == 0),
    }


# ==========================================================================
# v3.1 int8-residual mode (SquareQ README, "v3.1 - int8-residual mode"): the
# same format formula with an int8 residual that has one MSE-swept scale per
# output row, of the rotated residual left by a rank-16 split.  The page
# names the mode and nothing finer; these readings follow the W4 mode's
# stated sweep with the int8 grid:
#
#  W1 rank 16 (the page's number) through the same svd_init; any rank works.
#  W2 one scale per row of R (all K values): s_i = fp16(f_i a / 127), a the
#     row's absmax, f_i = (70 + i)/100 as in the W4 sweep, fp16 as R4.
#  W3 codes q = clamp(round_half_even(r / s), -128, 127) (the W4 grid's
#     asymmetric two's-complement range, one byte per code); zero scale -> 0.
#  W4 the first minimiser of the row's sum of squared errors wins (R6).
#  W5 codes are stored as int8 [N, K], scales as fp16 [N].
# ==========================================================================
W8_QMIN, W8_QMAX = -128, 127


def candidate_scale_exact_w8(absmax, i):
    """Unrounded candidate row scale f_i * absmax / 127 = (70+i)*absmax/12700 (fp64)."""
    return (70.0 + i) * np.asarray(absmax, np.float64) / 12700.0


def codes_for_scale_w8(r, s) -> np.ndarray:
    """Reading W3: q = clamp(round_half_even(r/s), -128, 127); q = 0 where s == 0."""
    r = np.asarray(r, np.float64)
    s = np.asarray(s, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(r / s), W8_QMIN, W8_QMAX)
    return np.where(s == 0, 0.0, q)


@dataclass
class QuantResultW8:
    q: np.ndarray        # int8 codes [N,K]
    scale: np.ndarray    # fp16 row scales [N] (float64 holding fp16 values)
    fidx: np.ndarray     # chosen fraction index [N] (uint8)
    mse: np.ndarray      # [N,31] sum of squared errors per candidate
    absmax: np.ndarray   # [N]


def quantize_residual_w8(r) -> QuantResultW8:
    """Sweep the 31 fractions once per row of the rotated residual (W2-W4)."""
    r = np.asarray(r, np.float64)
    n, k = r.shape
    if k % HBLOCK:
        raise ValueError("K must be a multiple of 256")
    if not np.all(np.isfinite(r)):
        raise FloatingPointError("non-finite residual")
    a = np.abs(r).max(axis=1)
    mse = np.empty((n, N_FRAC))
    scales = np.empty((n, N_FRAC))
    for i in range(N_FRAC):
        s = fp16_round(candidate_scale_exact_w8(a, i))
        if np.any(np.isinf(s)):
            raise FloatingPointError("fp16 scale overflow")
        q = codes_for_scale_w8(r, s[:, None])
        mse[:, i] = ((r - q * s[:, None]) ** 2).sum(axis=1)
        scales[:, i] = s
    best = np.argmin(mse, axis=1)          # the first minimum
    s_best = scales[np.arange(n), best]
    q_best = codes_for_scale_w8(r, s_best[:, None])
    return QuantResultW8(q_best.astype(np.int8), s_best, best.astype(np.uint8), mse, a)


def quantize_weight_w8(w, up, down) -> QuantResultW8:
    """Builder path of the int8 mode: residual against the bf16 factors, rotation, row sweep."""
    return quantize_residual_w8(residual(w, up, down))


def dequant_w8(q, scale) -> np.ndarray:
    """D = q * s_row (exact in fp64)."""
    return np.asarray(q, np.float64) * np.asarray(scale, np.float64)[:, None]


def reconstruct_w8(q, scale, up, down) -> np.ndarray:
    """W_hat = up @ down^T + rotate(dequant_w8(R)) in fp64 (format formula)."""
    lr = np.asarray(up, np.float64) @ np.asarray(down, np.float64).T
    return lr + rotate(dequant_w8(q, scale))


def forward_w8(x, q, scale, up, down) -> np.ndarray:
    """y = x @ W_hat^T = rotate(x) @ D^T + (x @ down) @ up^T in fp64."""
    x = np.asarray(x, np.float64)
    d = dequant_w8(q, scale)
    return rotate(x) @ d.T + (x @ np.asarray(down, np.float64)) @ np.asarray(up, np.float64).T


def forward_w8_fp16_operands(x, q, scale, up, down) -> np.ndarray:
    """Diagnostic forward: the activations rounded to fp16 as in
    forward_fp16_operands (row power of two 2^(11-E)); the codes are exact
    in fp16 and the row scale is applied to the exact product afterwards;
    the low-rank term is exact."""
    x = np.asarray(x, np.float64)
    xh = rotate(x)
    amax = np.abs(x).max(axis=1)
    e = np.zeros(x.shape[0])
    nz = amax > 0
    mant, ex = np.frexp(amax[nz])
    e[nz] = np.where(mant == 0.5, ex - 1, ex)
    f = np.ldexp(1.0, (11 - e).astype(np.int64))
    xh16 = fp16_round(xh * f[:, None])
    y = (xh16 @ np.asarray(q, np.float64).T) * np.asarray(scale, np.float64)[None, :] / f[:, None]
    return y + (x @ np.asarray(down, np.float64)) @ np.asarray(up, np.float64).T


def _variant_mse_w8(r, a):
    """Row errors of every candidate under each admissible fp16 rounding of
    its scale (variant 1 differs from variant 0 only within SCALE_MARGIN of
    a rounding boundary), as in _variant_mse."""
    n = r.shape[0]
    sc = np.empty((n, N_FRAC, 2))
    ms = np.empty((n, N_FRAC, 2))
    for i in range(N_FRAC):
        v = candidate_scale_exact_w8(a, i)
        s0 = fp16_round(v)
        lo, hi = _fp16_bracket(v)
        amb = _fp16_boundary_margin(v) <= SCALE_MARGIN
        s1 = np.where(amb, np.where(s0 == lo, hi, lo), s0)
        for j, sv in enumerate((s0, s1)):
            q = codes_for_scale_w8(r, sv[:, None])
            sc[:, i, j] = sv
            ms[:, i, j] = ((r - q * sv[:, None]) ** 2).sum(axis=1)
    return sc, ms


def certify_w8(r, res: QuantResultW8):
    """(rows, near): rows[n] is True where the row's scale choice is far from
    every tie (the chosen unrounded scale at least SCALE_MARGIN from an fp16
    rounding boundary and every other candidate's error above the best by
    SWEEP_MARGIN, under either admissible rounding); near[n, k] flags the
    values within CODE_MARGIN of a half-integer at the chosen scale, whose
    code a device residual that differs by fp32 rounding may take either
    way.  A row holds thousands of values, so codes are certified one by one
    rather than the whole row at once."""
    r = np.asarray(r, np.float64)
    a = res.absmax
    best = res.fidx.astype(np.int64)
    ok = _fp16_boundary_margin(candidate_scale_exact_w8(a, best)) > SCALE_MARGIN
    _, ms = _variant_mse_w8(r, a)
    others = ms.min(axis=-1)
    others[np.arange(len(best)), best] = np.inf
    mse_best = res.mse[np.arange(len(best)), best]
    ok &= others.min(axis=1) > mse_best * (1 + SWEEP_MARGIN)
    ok |= (a == 0)
    s = res.scale[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, r / np.where(s > 0, s, 1), 0.0)
    near = (np.abs(t - np.floor(t) - 0.5) < CODE_MARGIN) & (t > W8_QMIN - 1) & (t < W8_QMAX + 1)
    return ok, near


def check_device_quant_w8(r, res: QuantResultW8, q_dev, scale_dev, fidx_dev):
    """Compare a device int8-mode quantization with the oracle.

    Certified rows must have the oracle's index and scale bit for bit and its
    codes except at near-tie values (either neighbour).  Other rows must be
    admissible: the scale an admissible fp16 rounding for the device's index,
    the codes the requantization with that scale (near-ties either way), and
    the error within SWEEP_MARGIN of every other candidate's under its least
    favourable rounding.
    """
    r = np.asarray(r, np.float64)
    n, k = r.shape
    rows, near_o = certify_w8(r, res)
    qd = np.asarray(q_dev).astype(np.int64).reshape(n, k)
    qo = res.q.astype(np.int64)
    sd = np.asarray(scale_dev, np.float64).reshape(n)
    fd = np.asarray(fidx_dev).astype(np.int64).reshape(n)
    with np.errstate(divide="ignore", invalid="ignore"):
        t_o = np.where(res.scale[:, None] > 0, r / np.where(res.scale[:, None] > 0, res.scale[:, None], 1), 0.0)
    lo_o = np.clip(np.floor(t_o), W8_QMIN, W8_QMAX)
    hi_o = np.clip(np.ceil(t_o), W8_QMIN, W8_QMAX)
    codes_same = ((qd == qo) | (near_o & ((qd == lo_o) | (qd == hi_o)))).all(axis=1)
    same = (fd == res.fidx) & (sd == res.scale) & codes_same
    bad_cert = rows & ~same
    sc, ms = _variant_mse_w8(r, res.absmax)
    fdc = np.clip(fd, 0, N_FRAC - 1)
    cand = sc[np.arange(n), fdc]
    scale_ok = (sd == cand[:, 0]) | (sd == cand[:, 1])
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(sd[:, None] > 0, r / np.where(sd[:, None] > 0, sd[:, None], 1), 0.0)
    q_req = np.clip(np.rint(t), W8_QMIN, W8_QMAX)
    near = np.abs(t - np.floor(t) - 0.5) < CODE_MARGIN
    q_lo = np.clip(np.floor(t), W8_QMIN, W8_QMAX)
    q_hi = np.clip(np.ceil(t), W8_QMIN, W8_QMAX)
    codes_ok = ((qd == q_req) | (near & ((qd == q_lo) | (qd == q_hi)))).all(axis=1)
    mse_dev = ((r - qd * sd[:, None]) ** 2).sum(axis=1)
    worst = ms.max(axis=-1)
    worst[np.arange(n), fdc] = np.inf
    err_ok = mse_dev <= worst.min(axis=1) * (1 + SWEEP_MARGIN)
    err_ok |= (res.absmax == 0) & (mse_dev == 0)
    admissible = scale_ok & codes_ok & err_ok & (fd >= 0) & (fd < N_FRAC)
    bad_uncert = ~rows & ~same & ~admissible
    return {
        "rows": int(n),
        "uncertified": int((~rows).sum()),
        "differ": int((~same).sum()),
        "near_values": int(near_o.sum()),
        "bad_certified": int(bad_cert.sum()),
        "bad_uncertified": int(bad_uncert.sum()),
        "ok": bool(bad_cert.sum() == 0 and bad_uncert.sum() == 0),
    }


# ==========================================================================
# 4-bit float mode (the "Residual codecs" bullet's FP4 alternative: e2m1
# elements with block scales, driving native FP4 matrix instructions; the
# page's op-level parity line describes the forward as rotate + block-quant of
# the activations + FP4 product + epilogue).  The page's NVFP4 variant
# (ue4m3 block-16 scales, per-tensor scale, an NVIDIA tiled layout) exists
# for one vendor's instructions; the format here is its OCP MX counterpart,
# MXFP4, which the gfx950 scaled matrix instructions take.  Readings:
#
#  X1 element: FP4 E2M1 (1 sign, 2 exponent bits of bias 1, 1 mantissa bit):
#     magnitudes 0, 0.5 (the subnormal), 1, 1.5, 2, 3, 4, 6; nibble
#     s<<3 | e<<1 | m.  A value whose magnitude rounds to 0 gets nibble 0.
#  X2 block: 32 consecutive values along K share one E8M0 scale 2^(e-127).
#  X3 scale: e = floor(log2(absmax)) - 2 + 127 (2 = the largest E2M1
#     exponent), clamped to [0, 254]; an all-zero block gets e = 0.
#  X4 rounding: v / 2^(e-127) to the nearest E2M1 value, ties to the even
#     mantissa, magnitudes above 6 saturate to 6.
#  X5 operands: the rotated residual R of the W4 mode (same split, same
#     rotation) and the rotated activations x @ H, both quantized along K.
#  X6 forward: y = dq(Q(x H)) @ dq(Q(R))^T + (x @ down) @ up^T, the FP4 part
#     exact on the dequantized values (the device accumulates in fp32), the
#     low-rank part exact on the bf16 x.
#  X7 reconstruct: W_hat = up @ down^T + dq(Q(R)) @ H.
#  X8 packing: two nibbles per byte, even k in the low nibble (as R7);
#     scales one byte per block, [rows][K/32].
# ==========================================================================
MX_BLOCK = 32
E2M1_EMAX = 2


def e2m1_values() -> np.ndarray:
    """The 16 E2M1 code points by nibble (X1), from the format's definition:
    exponent field 0 is subnormal (m * 2^(1-1) * 0.5), otherwise
    2^(e-1) * (1 + m/2)."""
    out = np.empty(16)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
        out[c] = -mag if s else mag
    return out


def e2m1_encode(v) -> np.ndarray:
    """X1/X4: nearest E2M1 value of each fp64 v (ties to the even mantissa,
    saturating at 6); returns nibbles (uint8)."""
    v = np.asarray(v, np.float64)
    mags = e2m1_values()[:8]                       # nibbles 0..7, increasing
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - mags)                # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    tie = d == best
    # among equally near magnitudes take the even mantissa (nibble bit 0 clear)
    even = tie & ((np.arange(8) & 1) == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tie, axis=-1))
    code = np.where((v < 0) & (code != 0), code | 8, code)
    return code.astype(np.uint8)


def mx_scale_exponent(absmax) -> np.ndarray:
    """X3: E8M0 exponent byte of a block with the given absmax."""
    a = np.asarray(absmax, np.float64)
    e = np.zeros(a.shape, np.int64)
    nz = a > 0
    m, ex = np.frexp(a[nz])                        # a = m 2^ex, 0.5 <= m < 1
    e[nz] = (ex - 1) - E2M1_EMAX + 127             # floor(log2 a) = ex - 1
    return np.clip(e, 0, 254).astype(np.uint8)


def mx_quantize(a):
    """MXFP4 of rows of a [R,K] along K (X2-X4): (nibbles uint8 [R,K],
    exponent bytes uint8 [R,K/32])."""
    a = np.asarray(a, np.float64)
    r, k = a.shape
    if k % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    if not np.all(np.isfinite(a)):
        raise FloatingPointError("non-finite input")
    blocks = a.reshape(r, k // MX_BLOCK, MX_BLOCK)
    e = mx_scale_exponent(np.abs(blocks).max(axis=-1))
    x = np.ldexp(1.0, 127 - e.astype(np.int64))    # 1 / block scale (a power of two)
    codes = e2m1_encode(blocks * x[..., None]).reshape(r, k)
    return codes, e


def mx_dequant(codes, exps) -> np.ndarray:
    """value = E2M1(nibble) * 2^(e - 127), exact in fp64."""
    codes = np.asarray(codes, np.uint8)
    r, k = codes.shape
    v = e2m1_values()[codes].reshape(r, k // MX_BLOCK, MX_BLOCK)
    s = np.ldexp(1.0, np.asarray(exps).astype(np.int64) - 127)
    return (v * s[..., None]).reshape(r, k)


def mx_pack(codes) -> np.ndarray:
    """X8: two nibbles per byte, even k low."""
    c = np.asarray(codes).astype(np.int64)
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def mx_unpack(packed) -> np.ndarray:
    p = np.asarray(packed, np.uint8).astype(np.int64)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_weight_mx(w, up, down):
    """Builder of the FP4 mode (X5): MXFP4 of the rotated residual."""
    return mx_quantize(residual(w, up, down))


def quantize_act_mx(x):
    """Activation half of the FP4 forward (X5): MXFP4 of x @ H."""
    return mx_quantize(rotate(x))


def forward_mx(x, wcodes, wexps, up, down) -> np.ndarray:
    """X6 in fp64: the FP4 product on the dequantized operands plus the
    low-rank branch on the unquantized activations."""
    x = np.asarray(x, np.float64)
    xc, xe = quantize_act_mx(x)
    lr = (x @ np.asarray(down, np.float64)) @ np.asarray(up, np.float64).T
    return mx_dequant(xc, xe) @ mx_dequant(wcodes, wexps).T + lr


def reconstruct_mx(wcodes, wexps, up, down) -> np.ndarray:
    """X7 in fp64."""
    lr = np.asarray(up, np.float64) @ np.asarray(down, np.float64).T
    return lr + rotate(mx_dequant(wcodes, wexps))


MX_MARGIN = 1e-5     # relative distance from a rounding midpoint / a power of two


def _e2m1_midpoints() -> np.ndarray:
    m = e2m1_values()[:8]
    return (m[1:] + m[:-1]) / 2.0


def certify_mx(a, exps):
    """(blocks_ok [R,K/32], near [R,K]) for MXFP4 of a with the given exponents:
    a block is certified when its absmax is more than MX_MARGIN (relative)
    from a power of two (where fp32 rounding of the input could move the
    exponent); a value is near a tie when v / scale is within MX_MARGIN
    (relative) of a rounding midpoint, where either neighbour is admissible."""
    a = np.asarray(a, np.float64)
    r, k = a.shape
    blocks = a.reshape(r, k // MX_BLOCK, MX_BLOCK)
    am = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        l2 = np.log2(np.where(am > 0, am, 1.0))
    ok = (np.abs(l2 - np.rint(l2)) > MX_MARGIN / np.log(2)) | (am == 0)
    u = np.abs(blocks) * np.ldexp(1.0, 127 - np.asarray(exps).astype(np.int64))[..., None]
    mids = _e2m1_midpoints()
    near = (np.abs(u[..., None] - mids) <= MX_MARGIN * mids).any(axis=-1)
    return ok, near.reshape(r, k)


def check_device_mx(a, codes_dev, exps_dev):
    """Compare a device MXFP4 quantization of a [R,K] with the oracle's.

    Certified blocks must have the oracle's exponent and its nibbles except
    at near-tie values (either neighbour).  Other blocks must be admissible:
    the exponent one of the two a fp32 input could give (the oracle's or one
    off), and the nibbles the oracle's encoding under the device's exponent,
    near-ties either way.
    """
    a = np.asarray(a, np.float64)
    r, k = a.shape
    co, eo = mx_quantize(a)
    ok, near = certify_mx(a, eo)
    cd = np.asarray(codes_dev, np.uint8).reshape(r, k)
    ed = np.asarray(exps_dev, np.uint8).reshape(r, k // MX_BLOCK)
    vals = e2m1_values()

    def codes_match(e_used, c_dev, near_mask):
        ref = e2m1_encode(a * np.repeat(np.ldexp(1.0, 127 - e_used.astype(np.int64)), MX_BLOCK, axis=1))
        same = c_dev == ref
        # near a midpoint either neighbour: the device value must be one of the
        # two grid values around the exact one
        u = a * np.repeat(np.ldexp(1.0, 127 - e_used.astype(np.int64)), MX_BLOCK, axis=1)
        dv = vals[c_dev]
        mags = vals[:8]
        au = np.minimum(np.abs(u), 6.0)
        lo = mags[np.searchsorted(mags, au, side="right") - 1]
        hi = mags[np.minimum(np.searchsorted(mags, au, side="left"), 7)]
        nb = (np.abs(dv) == lo) | (np.abs(dv) == hi)
        sign_ok = (dv == 0) | (np.sign(dv) == np.sign(u))
        return (same | (near_mask & nb & sign_ok)).reshape(r, k // MX_BLOCK, MX_BLOCK).all(axis=-1)

    cert_same = (ed == eo) & codes_match(eo, cd, near)
    bad_cert = ok & ~cert_same
    _, near_d = certify_mx(a, ed)
    adm = (np.abs(ed.astype(np.int64) - eo.astype(np.int64)) <= 1) & codes_match(ed, cd, near_d)
    bad_uncert = ~ok & ~cert_same & ~adm
    return {
        "blocks": int(ok.size),
        "uncertified": int((~ok).sum()),
        "differ": int((~cert_same).sum()),
        "near_values": int(near.sum()),
        "bad_certified": int(bad_cert.sum()),
        "bad_uncertified": int(bad_uncert.sum()),
        "ok": bool(bad_cert.sum() == 0 and bad_uncert.sum() == 0),
    }
