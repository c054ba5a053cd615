"""Shared helpers of the device parity tests (host side only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from synth import CONFIGS, gen_layer, gen_payload


def dev():
    return torch.device("cuda:0")


def to_dev_payload(codes, scales, up_bits, down_bits, group):
    """numpy payload (uint8 codes, fp16 scales, bf16 bits) -> W4Payload on the GPU."""
    from w4_gemm_amd import W4Payload
    d = dev()
    up_bits = None if up_bits is None else np.ascontiguousarray(up_bits)
    down_bits = None if down_bits is None else np.ascontiguousarray(down_bits)
    up = torch.from_numpy(up_bits.view(np.int16)).view(torch.bfloat16).to(d) if up_bits is not None else None
    dn = torch.from_numpy(down_bits.view(np.int16)).view(torch.bfloat16).to(d) if down_bits is not None else None
    return W4Payload(torch.from_numpy(codes).to(d), torch.from_numpy(scales).to(d), up, dn, group)


def bf16_bits_of(a64: np.ndarray) -> np.ndarray:
    """fp64 array holding bf16 values -> bf16 bit patterns (exact)."""
    a = np.ascontiguousarray(a64, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def payload_fp64(codes, scales, up_bits, down_bits):
    q = O.unpack(codes).astype(np.float64)
    s = O.fp16_decode(np.asarray(scales))
    up = O.bf16_decode(up_bits) if up_bits is not None else np.zeros((codes.shape[0], 0))
    dn = O.bf16_decode(down_bits) if down_bits is not None else np.zeros((codes.shape[1] * 2, 0))
    return q, s, up, dn


def oracle_payload(w, rank, group):
    """Oracle quantization of W with its own SVD split -> (numpy payload, QuantResult, R)."""
    up, dn = O.svd_init(w, rank)
    r = O.residual(w, up, dn)
    res = O.quantize_residual(r, group)
    codes = O.pack(res.q)
    scales = res.scale.astype(np.float16)
    return (codes, scales, bf16_bits_of(up) if rank else None, bf16_bits_of(dn) if rank else None,
            res, r, up, dn)


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |a| (a holds bf16 values)."""
    m, e = np.frexp(np.abs(a))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)
