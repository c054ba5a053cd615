"""Shape checks of the torch-facing wrappers, as pure functions of shapes.

The C ABI (include/sq.h) takes raw device pointers and derives every extent
from the sizes it is given, so a tensor whose shape disagrees with them would
be read or written past its end on the device.  The wrappers in api.py call
these checks before any pointer reaches the library; each raises ValueError
naming the tensor and the shape it must have.  Kept free of torch so that the
host tests exercise them without a GPU.
"""
from __future__ import annotations


def _shape(s) -> tuple:
    return tuple(int(v) for v in s)


def _need(name: str, got, want) -> None:
    got, want = _shape(got), _shape(want)
    if got != want:
        raise ValueError(f"{name} must have shape {list(want)}, got {list(got)}")


def _factors(n: int, k: int, up, down, ranks) -> int:
    """up [n, r] and down [k, r], both present or both absent; returns r."""
    if (up is None) != (down is None):
        raise ValueError("lora_up and lora_down must both be given or both be None")
    if up is None:
        return 0
    up, down = _shape(up), _shape(down)
    if len(up) != 2 or len(down) != 2:
        raise ValueError("lora_up and lora_down must be 2-D")
    r = up[1]
    _need("lora_up", up, (n, r))
    _need("lora_down", down, (k, r))
    if r not in ranks:
        raise ValueError(f"rank must be one of {sorted(ranks)}, got {r}")
    return r


def check_w4_payload(codes, scales, up, down, group: int) -> tuple:
    """W4 payload: codes u8 [N, K/2], scales fp16 [N, K/group], up [N, r], down [K, r].

    Returns (n, k, rank).  K is twice the codes' row length; it must be a
    positive multiple of 256, group 32 or 64 and rank 0, 32 or 64.
    """
    codes = _shape(codes)
    if len(codes) != 2:
        raise ValueError("codes must be 2-D [N, K/2]")
    n, k = codes[0], 2 * codes[1]
    if n < 1 or k < 256 or k % 256:
        raise ValueError(f"need N >= 1 and K a positive multiple of 256, got N={n} K={k}")
    if group not in (32, 64):
        raise ValueError(f"group must be 32 or 64, got {group}")
    _need("scales", scales, (n, k // group))
    r = _factors(n, k, up, down, (32, 64))
    return n, k, r


def check_w8_payload(codes, scales, up, down) -> tuple:
    """int8-residual payload: codes i8 [N, K], scales fp16 [N], up [N, r], down [K, r]."""
    codes = _shape(codes)
    if len(codes) != 2:
        raise ValueError("codes must be 2-D [N, K]")
    n, k = codes
    if n < 1 or k < 256 or k % 256:
        raise ValueError(f"need N >= 1 and K a positive multiple of 256, got N={n} K={k}")
    _need("scales", scales, (n,))
    r = _factors(n, k, up, down, (16, 32, 64))
    return n, k, r


def check_mx4_payload(codes, exps, up, down) -> tuple:
    """MXFP4 payload: codes u8 [N, K/2], exps u8 [N, K/32], up [N, r], down [K, r]."""
    codes = _shape(codes)
    if len(codes) != 2:
        raise ValueError("codes must be 2-D [N, K/2]")
    n, k = codes[0], 2 * codes[1]
    if n < 1 or k < 256 or k % 256:
        raise ValueError(f"need N >= 1 and K a positive multiple of 256, got N={n} K={k}")
    _need("exps", exps, (n, k // 32))
    r = _factors(n, k, up, down, (16, 32, 64))
    return n, k, r


def check_rows(name: str, a, cols: int) -> int:
    """a must be 2-D [M, cols]; returns M."""
    a = _shape(a)
    if len(a) != 2 or a[1] != cols:
        raise ValueError(f"{name} must be 2-D [M, {cols}], got {list(a)}")
    return a[0]


def check_out(name: str, out, shape) -> None:
    _need(name, out, shape)


def check_weight(w, up, down, ranks=(32, 64)) -> tuple:
    """Quantizer input: w fp32 [N, K] with K a positive multiple of 256, factors as above."""
    w = _shape(w)
    if len(w) != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w
    if n < 1 or k < 256 or k % 256:
        raise ValueError(f"need N >= 1 and K a positive multiple of 256, got N={n} K={k}")
    r = _factors(n, k, up, down, ranks)
    return n, k, r
