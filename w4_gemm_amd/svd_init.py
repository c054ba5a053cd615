"""Host step before the quantizer: the rank-r low-rank branch of a weight.

SquareQ README, "SquareQ v3 - W4", "Low-rank branch" bullet: a rank-32 SVD of
the weight, always on, stored in bf16.  The split puts sqrt of the singular
values on both sides (up = U_r sqrt(S_r), down = V_r sqrt(S_r)) and rounds
each factor to bf16 once, from fp64.  Runs on the host in fp64 LAPACK; there
is no device SVD kernel.
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16_from_f64(a: np.ndarray) -> torch.Tensor:
    """Round fp64 to bf16 (nearest even) in one step, via integer bit arithmetic.

    fp64 -> bf16 through fp32 would round twice; instead the fp64 bit pattern
    is rounded at bf16's 8-bit significand directly.  Values here are normal
    and far from the bf16 range limits.
    """
    a = np.ascontiguousarray(a, dtype=np.float64)
    bits = a.view(np.uint64)
    # fp64 has 52 fraction bits, bf16 keeps 7: drop 45 with round-half-even
    drop = 45
    half = np.uint64(1) << np.uint64(drop - 1)
    lsb = (bits >> np.uint64(drop)) & np.uint64(1)
    rounded = (bits + half - np.uint64(1) + lsb) >> np.uint64(drop)
    sign = (rounded >> np.uint64(18)) & np.uint64(1)
    exp = (rounded >> np.uint64(7)) & np.uint64(0x7FF)
    frac = rounded & np.uint64(0x7F)
    e8 = exp.astype(np.int64) - 1023 + 127
    zero = (exp == 0)
    out = (sign << np.uint64(15)) | (np.clip(e8, 0, 255).astype(np.uint64) << np.uint64(7)) | frac
    out = np.where(zero, sign << np.uint64(15), out).astype(np.uint16)
    return torch.from_numpy(out.view(np.int16).copy()).view(torch.bfloat16)


def svd_init(w, rank: int = 32):
    """(up [N,rank], down [K,rank]) as bf16 CPU tensors from an fp32/fp64 weight."""
    w = np.asarray(w.cpu().numpy() if isinstance(w, torch.Tensor) else w, dtype=np.float64)
    if rank == 0:
        return None, None
    u, s, vt = np.linalg.svd(w, full_matrices=False)
    r = np.sqrt(s[:rank])
    return _bf16_from_f64(u[:, :rank] * r), _bf16_from_f64(vt[:rank].T * r)
