"""Seeded synthetic inputs for the W4 linear layer.

This module is shared by the oracle tests and the device tests.  It holds
no part of the layer's arithmetic: it only draws random weights,
activations and (for large-shape device tests) random payloads, and it
encodes fp32 draws as bf16 bit patterns.

Workload recipe (SquareQ README, "SquareQ v3 - W4" section: the layer
shapes of the NVFP4-vs-bf16 table and the int4 group-32/64 codec):

* W  = N(0,1)[N,K]/sqrt(K) + U diag(sigma) V^T, U,V orthonormal bases of a
  rank-s spike, sigma = linspace(8, 2, s); cast to fp32.
* x  = N(0,1)[M,K] with round(p*K) outlier channels multiplied by 20,
  rounded to bf16 (round-to-nearest-even).
* draws happen in that order from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    N: int
    K: int
    group: int
    rank: int
    spike: int
    outlier_frac: float
    small_m: tuple = ()


# The five layer shapes: a tiny layer, an attention projection, a fused QKV
# projection, an MLP-up and an MLP-down (long K) projection.
CONFIGS = {
    1: LayerConfig("tiny 64x512x512 g32", 64, 512, 512, 32, 32, 4, 0.01),
    2: LayerConfig("attn-proj 1536x3072x3072 g32", 1536, 3072, 3072, 32, 32, 8, 0.005),
    3: LayerConfig("fused-qkv 1536x9216x3072 g64", 1536, 9216, 3072, 64, 32, 8, 0.005),
    4: LayerConfig("mlp-up 4480x16384x6144 g32", 4480, 16384, 6144, 32, 32, 8, 0.005),
    5: LayerConfig("mlp-down 4480x6144x16384 g32", 4480, 6144, 16384, 32, 32, 8, 0.005,
                   small_m=(1, 16, 32, 64, 128)),
}


def f32_to_bf16_bits(a) -> np.ndarray:
    """Encode fp32 values as bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite draws; NaN handling is not needed here.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_weight_parts(rng: np.random.Generator, N: int, K: int, spike: int):
    """(W fp32 [N,K], U [N,s], sigma [s], V [K,s]): the weight of ``gen_weight``
    together with its planted rank-``spike`` component U diag(sigma) V^T."""
    g = rng.standard_normal((N, K)) / np.sqrt(K)
    u = np.linalg.qr(rng.standard_normal((N, spike)))[0]
    v = np.linalg.qr(rng.standard_normal((K, spike)))[0]
    sig = np.linspace(8.0, 2.0, spike)
    w = g + (u * sig) @ v.T
    return w.astype(np.float32), u, sig, v


def gen_weight(rng: np.random.Generator, N: int, K: int, spike: int) -> np.ndarray:
    """W fp32 [N,K]: N(0,1/K) bulk plus a rank-``spike`` component, sigma 8..2."""
    return gen_weight_parts(rng, N, K, spike)[0]


def gen_activations(rng: np.random.Generator, M: int, K: int, outlier_frac: float) -> np.ndarray:
    """x as bf16 bits [M,K]: N(0,1) with round(p*K) channels scaled by 20."""
    x = rng.standard_normal((M, K))
    n_out = int(round(outlier_frac * K))
    if n_out:
        idx = rng.choice(K, n_out, replace=False)
        x[:, idx] *= 20.0
    return f32_to_bf16_bits(x.astype(np.float32))


def gen_layer(cfg_id: int, seed: int = 0, with_x: bool = True):
    """(cfg, W fp32 [N,K], x bf16 bits [M,K] or None) for one of the five shapes."""
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng(seed)
    w = gen_weight(rng, cfg.N, cfg.K, cfg.spike)
    x = gen_activations(rng, cfg.M, cfg.K, cfg.outlier_frac) if with_x else None
    return cfg, w, x


def gen_payload(rng: np.random.Generator, N: int, K: int, group: int, rank: int):
    """A random W4 payload with the statistics of a quantized N(0,1/K) weight.

    Used where building the payload through the full sweep would take the
    CPU too long (the 100M-element shapes).  Returns packed codes uint8
    [N,K/2], fp16 scales [N,K/group], bf16 bits of up [N,rank] and
    down [K,rank].

    Codes follow a clipped rounded normal (|q| = 7 common at group maxima);
    scales are drawn around the typical f*absmax/7 of such a weight.
    """
    q = np.clip(np.rint(rng.standard_normal((N, K)) * 3.5), -8, 7).astype(np.int8)
    lo = (q[:, 0::2].astype(np.uint8) & 0xF)
    hi = (q[:, 1::2].astype(np.uint8) & 0xF)
    codes = (lo | (hi << 4)).astype(np.uint8)
    base = 1.8 / np.sqrt(K) / 7.0
    scales = (base * np.exp(0.15 * rng.standard_normal((N, K // group)))).astype(np.float16)
    up = f32_to_bf16_bits((rng.standard_normal((N, rank)) * (1.5 / np.sqrt(N))).astype(np.float32))
    down = f32_to_bf16_bits((rng.standard_normal((K, rank)) * (1.5 / np.sqrt(K))).astype(np.float32))
    return codes, scales, up, down


def gen_payload_w8(rng: np.random.Generator, N: int, K: int, rank: int):
    """A random int8-residual payload with the statistics of a quantized
    N(0,1/K) weight: int8 codes [N,K] from a clipped rounded normal of
    spread 30, fp16 row scales around 4.5/sqrt(K)/127, bf16 bits of up
    [N,rank] and down [K,rank]."""
    q = np.clip(np.rint(rng.standard_normal((N, K)) * 30.0), -128, 127).astype(np.int8)
    base = 4.5 / np.sqrt(K) / 127.0
    scales = (base * np.exp(0.1 * rng.standard_normal(N))).astype(np.float16)
    up = f32_to_bf16_bits((rng.standard_normal((N, rank)) * (1.5 / np.sqrt(N))).astype(np.float32))
    down = f32_to_bf16_bits((rng.standard_normal((K, rank)) * (1.5 / np.sqrt(K))).astype(np.float32))
    return q, scales, up, down


def gen_payload_mx(rng: np.random.Generator, N: int, K: int, rank: int):
    """A random MXFP4 payload: uniform E2M1 nibbles packed two per byte
    [N,K/2], E8M0 block exponents around those of an N(0,1/K) weight
    (120 +- 1 at K = 6144, shifted with log2 K) [N,K/32], bf16 bits of up
    [N,rank] and down [K,rank]."""
    nib = rng.integers(0, 16, (N, K), dtype=np.uint8)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    base = int(round(127 - 2 - 0.5 * np.log2(K) + 1.3))
    exps = (base + rng.integers(-1, 2, (N, K // 32))).astype(np.uint8)
    up = f32_to_bf16_bits((rng.standard_normal((N, rank)) * (1.5 / np.sqrt(N))).astype(np.float32))
    down = f32_to_bf16_bits((rng.standard_normal((K, rank)) * (1.5 / np.sqrt(K))).astype(np.float32))
    return codes, exps, up, down
