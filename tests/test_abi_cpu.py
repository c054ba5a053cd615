"""Host-side checks of libsq that need no GPU: the library loads, exports every
symbol include/sq.h declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

from w4_gemm_amd import _lib
from w4_gemm_amd._lib import SqW4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    L = _lib.lib()
    for name in names:
        assert hasattr(L, name), name
    # and they are real dynamic symbols of libsq.so
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in names:
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_status_strings():
    assert _lib.abi_version() == 1
    for s in range(10):
        assert _lib.status_str(s)
    assert "unknown" in _lib.status_str(99)


def _payload(n=16, k=256, group=32, rank=32, codes=0x1000, scales=0x2000, up=0x3000, down=0x4000):
    return SqW4(n, k, group, rank, codes, scales, up, down)


BAD = [
    ("k not multiple of 256", dict(k=300), 2),
    ("k too small", dict(k=0), 2),
    ("n < 1", dict(n=0), 2),
    ("group 16", dict(group=16), 3),
    ("rank 16", dict(rank=16), 4),
    ("null codes", dict(codes=None), 1),
    ("null up with rank", dict(up=None), 1),
    ("misaligned scales", dict(scales=0x2002), 5),
]


@pytest.mark.parametrize("why,kw,status", BAD, ids=[b[0] for b in BAD])
def test_validation_before_launch(why, kw, status):
    p = _payload(**kw)
    assert _lib.sq_reconstruct_bf16(p, 0x5000, None) == status
    assert _lib.sq_quantize_weight(0x6000, p, None, 0x7000, None) == status
    assert _lib.sq_linear_fwd(0x8000, 4, p, 0x9000, 0, 0xA000, 1 << 30, None) == status
    assert _lib.sq_linear_dgrad(0x8000, 4, p, 0x9000, 0, 0xA000, 1 << 30, None) == status


def test_other_arguments():
    p = _payload()
    assert _lib.sq_reconstruct_bf16(p, None, None) == 1
    assert _lib.sq_reconstruct_bf16(p, 0x5008, None) == 5
    assert _lib.sq_quantize_weight(None, p, None, 0x7000, None) == 1
    assert _lib.sq_quantize_weight(0x6000, p, None, None, None) == 1
    assert _lib.sq_linear_fwd(0x8000, -1, p, 0x9000, 0, 0xA000, 1 << 30, None) == 2
    assert _lib.sq_linear_fwd(0x8000, 4, p, 0x9000, 7, 0xA000, 1 << 30, None) == 7
    assert _lib.sq_linear_fwd(0x8000, 0, p, 0x9000, 0, None, 0, None) == 0   # m == 0: no-op
    ws = _lib.sq_linear_fwd_workspace_bytes(4, p)
    assert _lib.sq_linear_fwd(0x8000, 4, p, 0x9000, 0, 0xA000, ws - 1, None) == 6
    # rank 0 needs no factors
    p0 = _payload(rank=0, up=None, down=None)
    assert _lib.sq_linear_fwd_workspace_bytes(4, p0) > 0


def test_dgrad_arguments():
    p = _payload(n=128)
    big = 1 << 40
    assert _lib.sq_linear_dgrad(0x8000, 4, _payload(n=16), 0x9000, 0, 0xA000, big, None) == 2
    assert _lib.sq_linear_dgrad_workspace_bytes(4, _payload(n=16)) == 0
    assert _lib.sq_linear_dgrad(0x8000, -1, p, 0x9000, 0, 0xA000, big, None) == 2
    assert _lib.sq_linear_dgrad(0x8000, 4, p, 0x9000, 7, 0xA000, big, None) == 7
    assert _lib.sq_linear_dgrad(0x8000, 0, p, 0x9000, 0, None, 0, None) == 0   # m == 0: no-op
    assert _lib.sq_linear_dgrad(None, 4, p, 0x9000, 0, 0xA000, big, None) == 1
    assert _lib.sq_linear_dgrad(0x8000, 4, p, None, 0, 0xA000, big, None) == 1
    assert _lib.sq_linear_dgrad(0x8008, 4, p, 0x9000, 0, 0xA000, big, None) == 5
    ws = _lib.sq_linear_dgrad_workspace_bytes(4, p)
    assert ws >= 4 * 256 * 4                          # holds the fp32 accumulator
    assert _lib.sq_linear_dgrad(0x8000, 4, p, 0x9000, 0, 0xA000, ws - 1, None) == 6
    p0 = _payload(n=128, rank=0, up=None, down=None)
    assert 0 < _lib.sq_linear_dgrad_workspace_bytes(4, p0) < ws


def test_workspace_size_grows_with_m():
    p = _payload(n=3072, k=3072)
    sizes = [_lib.sq_linear_fwd_workspace_bytes(m, p) for m in (1, 64, 1536)]
    assert sizes[0] > 0 and sizes[0] <= sizes[1] <= sizes[2]
    assert sizes[2] >= 1536 * 3072 * 2                 # holds the rotated activations
    assert _lib.sq_linear_fwd_workspace_bytes(0, p) == 0


# ------------------------------------------------------------------ int8-residual mode
def _payload_w8(n=16, k=256, rank=16, reserved=0, codes=0x1000, scales=0x2000, up=0x3000,
                down=0x4000):
    return _lib.SqW8(n, k, rank, reserved, codes, scales, up, down)


BAD_W8 = [
    ("k not multiple of 256", dict(k=300), 2),
    ("n < 1", dict(n=0), 2),
    ("rank 8", dict(rank=8), 4),
    ("reserved set", dict(reserved=1), 4),
    ("null codes", dict(codes=None), 1),
    ("null scales", dict(scales=None), 1),
    ("null down with rank", dict(down=None), 1),
    ("misaligned codes", dict(codes=0x1004), 5),
]


@pytest.mark.parametrize("why,kw,status", BAD_W8, ids=[b[0] for b in BAD_W8])
def test_w8_validation_before_launch(why, kw, status):
    p = _payload_w8(**kw)
    big = 1 << 40
    assert _lib.sq_reconstruct_bf16_w8(p, 0x5000, None) == status
    assert _lib.sq_quantize_weight_w8(0x6000, p, None, 0x7000, 0xB000, big, None) == status
    assert _lib.sq_linear_fwd_w8(0x8000, 4, p, 0x9000, 0, 0xA000, big, None) == status


def test_w8_other_arguments():
    p = _payload_w8()
    big = 1 << 40
    for rank in (0, 16, 32, 64):
        pr = _payload_w8(rank=rank, up=None if rank == 0 else 0x3000,
                         down=None if rank == 0 else 0x4000)
        assert _lib.sq_linear_fwd_w8_workspace_bytes(4, pr) > 0
    qws = _lib.sq_quantize_weight_w8_workspace_bytes(p)
    assert qws >= 16 * 256 * 4                        # holds the fp32 rotated residual
    assert _lib.sq_quantize_weight_w8(0x6000, p, None, 0x7000, 0xB000, qws - 1, None) == 6
    assert _lib.sq_quantize_weight_w8(0x6000, p, None, 0x7000, None, qws, None) == 1
    assert _lib.sq_quantize_weight_w8(0x6000, p, 0x7008, 0x7000, 0xB000, qws, None) == 5
    assert _lib.sq_linear_fwd_w8(0x8000, 0, p, 0x9000, 0, None, 0, None) == 0   # m == 0: no-op
    assert _lib.sq_linear_fwd_w8(0x8000, -1, p, 0x9000, 0, 0xA000, big, None) == 2
    assert _lib.sq_linear_fwd_w8(0x8000, 4, p, 0x9000, 7, 0xA000, big, None) == 7
    ws = _lib.sq_linear_fwd_w8_workspace_bytes(4, p)
    assert _lib.sq_linear_fwd_w8(0x8000, 4, p, 0x9000, 0, 0xA000, ws - 1, None) == 6
    assert _lib.sq_reconstruct_bf16_w8(p, None, None) == 1


# ------------------------------------------------------------------ MXFP4 mode
def _payload_mx(n=16, k=256, rank=32, reserved=0, codes=0x1000, exps=0x2000, up=0x3000,
                down=0x4000):
    return _lib.SqMx4(n, k, rank, reserved, codes, exps, up, down)


BAD_MX = [
    ("k not multiple of 256", dict(k=288), 2),
    ("n < 1", dict(n=0), 2),
    ("rank 48", dict(rank=48), 4),
    ("reserved set", dict(reserved=2), 4),
    ("null codes", dict(codes=None), 1),
    ("null exps", dict(exps=None), 1),
    ("null up with rank", dict(up=None), 1),
    ("misaligned exps", dict(exps=0x2001), 5),
]


@pytest.mark.parametrize("why,kw,status", BAD_MX, ids=[b[0] for b in BAD_MX])
def test_mx_validation_before_launch(why, kw, status):
    p = _payload_mx(**kw)
    big = 1 << 40
    assert _lib.sq_reconstruct_bf16_mx4(p, 0x5000, None) == status
    assert _lib.sq_quantize_weight_mx4(0x6000, p, 0x7000, None) == status
    assert _lib.sq_linear_fwd_mx4(0x8000, 4, p, 0x9000, 0, 0xA000, big, None) == status


def test_mx_other_arguments():
    p = _payload_mx()
    big = 1 << 40
    assert _lib.sq_quantize_weight_mx4(None, p, 0x7000, None) == 1
    assert _lib.sq_quantize_weight_mx4(0x6000, p, None, None) == 1
    assert _lib.sq_quantize_act_mx4(0x8000, 4, 300, 0x9000, 0xA000, None) == 2
    assert _lib.sq_quantize_act_mx4(0x8000, -1, 256, 0x9000, 0xA000, None) == 2
    assert _lib.sq_quantize_act_mx4(0x8000, 0, 256, None, None, None) == 0   # m == 0: no-op
    assert _lib.sq_quantize_act_mx4(0x8000, 4, 256, None, 0xA000, None) == 1
    assert _lib.sq_quantize_act_mx4(0x8000, 4, 256, 0x9004, 0xA000, None) == 5
    assert _lib.sq_linear_fwd_mx4(0x8000, 0, p, 0x9000, 0, None, 0, None) == 0   # m == 0: no-op
    assert _lib.sq_linear_fwd_mx4(0x8000, -1, p, 0x9000, 0, 0xA000, big, None) == 2
    assert _lib.sq_linear_fwd_mx4(0x8000, 4, p, 0x9000, 9, 0xA000, big, None) == 7
    ws = _lib.sq_linear_fwd_mx4_workspace_bytes(4, p)
    assert ws >= 4 * 128 + 4 * 8                      # holds the FP4 activations and exponents
    assert _lib.sq_linear_fwd_mx4(0x8000, 4, p, 0x9000, 0, 0xA000, ws - 1, None) == 6
    assert _lib.sq_reconstruct_bf16_mx4(p, None, None) == 1
    for rank in (0, 16, 32, 64):
        pr = _payload_mx(rank=rank, up=None if rank == 0 else 0x3000,
                         down=None if rank == 0 else 0x4000)
        assert _lib.sq_linear_fwd_mx4_workspace_bytes(4, pr) > 0


def test_static_forward_arguments():
    # validation and the scratch limit come before any HIP call
    p = _payload()
    assert _lib.sq_linear_fwd_static(0x8000, 0, p, 0x9000, 0, None) == 0      # m == 0: no-op
    assert _lib.sq_linear_fwd_static(0x8000, -1, p, 0x9000, 0, None) == 2
    assert _lib.sq_linear_fwd_static(0x8000, 4, p, 0x9000, 5, None) == 7
    assert _lib.sq_linear_fwd_static(None, 4, p, 0x9000, 0, None) == 1
    assert _lib.sq_linear_fwd_static(0x8000, 4, p, 0x9008, 0, None) == 5
    assert _lib.sq_linear_fwd_static(0x8000, 4, _payload(rank=16), 0x9000, 0, None) == 4
    big = _payload(n=6144, k=16384)                   # 4480 rows need ~146 MB of scratch
    assert _lib.sq_linear_fwd_workspace_bytes(4480, big) > _lib.SQ_FWD_STATIC_SCRATCH_BYTES
    assert _lib.sq_linear_fwd_static(0x8000, 4480, big, 0x9000, 0, None) == 6
    head = _payload(n=16384, k=6144)
    assert _lib.sq_linear_fwd_workspace_bytes(4480, head) <= _lib.SQ_FWD_STATIC_SCRATCH_BYTES
    for m in (1, 16):
        assert _lib.sq_linear_fwd_workspace_bytes(m, big) <= _lib.SQ_FWD_STATIC_SCRATCH_BYTES
