"""Thin torch-facing wrappers over the C ABI (include/sq.h).

PyTorch only allocates device memory and supplies the current HIP stream;
every step of the layer runs in libsq's kernels.  Each call raises SqError on a
non-OK status.  Tensors must live on the current device.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib
from . import shapes as S
from ._lib import SqError, SqMx4, SqW4, SqW8, SQ_BF16, SQ_F32


@dataclass
class W4Payload:
    """Device tensors of one W4 layer (layouts as in sq.h)."""
    codes: torch.Tensor      # uint8 [N, K/2]
    scales: torch.Tensor     # float16 [N, K/group]
    up: torch.Tensor | None  # bfloat16 [N, rank]
    down: torch.Tensor | None  # bfloat16 [K, rank]
    group: int

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1] * 2

    @property
    def rank(self) -> int:
        return 0 if self.up is None else self.up.shape[1]

    def abi(self) -> SqW4:
        _require(self.codes, torch.uint8, "codes")
        _require(self.scales, torch.float16, "scales")
        S.check_w4_payload(self.codes.shape, self.scales.shape, _shp(self.up), _shp(self.down),
                           self.group)
        if self.up is not None:
            _require(self.up, torch.bfloat16, "up")
            _require(self.down, torch.bfloat16, "down")
        return SqW4(self.n, self.k, self.group, self.rank, _ptr(self.codes), _ptr(self.scales),
                    _ptr(self.up), _ptr(self.down))


def _require(t, dtype, name):
    """The C ABI takes dense row-major device buffers: refuse anything else."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _shp(t):
    return None if t is None else tuple(t.shape)


def _nbytes(t):
    """Byte size of a caller's workspace tensor (dense, on the device)."""
    _require(t, t.dtype, "workspace")
    return t.numel() * t.element_size()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != _lib.SQ_OK:
        raise SqError(status, where)


def empty_payload(n: int, k: int, group: int, rank: int, device="cuda") -> W4Payload:
    up = torch.empty((n, rank), dtype=torch.bfloat16, device=device) if rank else None
    down = torch.empty((k, rank), dtype=torch.bfloat16, device=device) if rank else None
    return W4Payload(torch.empty((n, k // 2), dtype=torch.uint8, device=device),
                     torch.empty((n, k // group), dtype=torch.float16, device=device),
                     up, down, group)


def quantize_weight(w: torch.Tensor, up: torch.Tensor | None, down: torch.Tensor | None,
                    group: int, want_fidx: bool = True):
    """sq_quantize_weight: fp32 W [N,K] and bf16 factors -> (payload, fidx, flags tensor)."""
    _require(w, torch.float32, "w")
    n, k, rank = S.check_weight(w.shape, _shp(up), _shp(down))
    p = empty_payload(n, k, group, rank, w.device)
    p.up, p.down = up, down
    fidx = torch.empty((n, k // group), dtype=torch.uint8, device=w.device) if want_fidx else None
    flags = torch.zeros(4, dtype=torch.int32, device=w.device)
    _check(_lib.sq_quantize_weight(w.data_ptr(), p.abi(), _ptr(fidx), flags.data_ptr(), _stream()),
           "sq_quantize_weight")
    return p, fidx, flags


def fwd_workspace_bytes(m: int, p: W4Payload) -> int:
    return _lib.sq_linear_fwd_workspace_bytes(m, p.abi())


def linear_fwd(x: torch.Tensor, p: W4Payload, out_dtype=torch.float32,
               workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """sq_linear_fwd: bf16 x [M,K] -> y [M,N] (fp32 or bf16)."""
    _require(x, torch.bfloat16, "x")
    m = S.check_rows("x", x.shape, p.k)
    if out is None:
        out = torch.empty((m, p.n), dtype=out_dtype, device=x.device)
    _require(out, out.dtype, "out")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, p.n):
        raise ValueError("out must be fp32 or bf16 of shape [M, N]")
    dt = SQ_BF16 if out.dtype == torch.bfloat16 else SQ_F32
    nbytes = fwd_workspace_bytes(m, p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check(_lib.sq_linear_fwd(x.data_ptr(), m, p.abi(), out.data_ptr(), dt, workspace.data_ptr(),
                              _nbytes(workspace), _stream()), "sq_linear_fwd")
    return out


def linear_fwd_static(x: torch.Tensor, p: W4Payload, out_dtype=torch.float32,
                      out: torch.Tensor | None = None):
    """sq_linear_fwd_static: the forward with the library's static scratch (no workspace)."""
    _require(x, torch.bfloat16, "x")
    m = S.check_rows("x", x.shape, p.k)
    if out is None:
        out = torch.empty((m, p.n), dtype=out_dtype, device=x.device)
    _require(out, out.dtype, "out")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, p.n):
        raise ValueError("out must be fp32 or bf16 of shape [M, N]")
    dt = SQ_BF16 if out.dtype == torch.bfloat16 else SQ_F32
    _check(_lib.sq_linear_fwd_static(x.data_ptr(), m, p.abi(), out.data_ptr(), dt, _stream()),
           "sq_linear_fwd_static")
    return out


def linear_fwd_rotate(x: torch.Tensor, p: W4Payload, workspace: torch.Tensor):
    """sq_linear_fwd_rotate: the activation half of the forward, into `workspace`."""
    _require(x, torch.bfloat16, "x")
    S.check_rows("x", x.shape, p.k)
    _check(_lib.sq_linear_fwd_rotate(x.data_ptr(), x.shape[0], p.abi(), workspace.data_ptr(),
                                     _nbytes(workspace), _stream()),
           "sq_linear_fwd_rotate")


def linear_fwd_contract(m: int, p: W4Payload, out: torch.Tensor, workspace: torch.Tensor):
    """sq_linear_fwd_contract: the weight half of the forward, from `workspace` into out."""
    _require(out, out.dtype, "out")
    S.check_out("out", out.shape, (m, p.n))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out must be fp32 or bf16")
    dt = SQ_BF16 if out.dtype == torch.bfloat16 else SQ_F32
    _check(_lib.sq_linear_fwd_contract(m, p.abi(), out.data_ptr(), dt, workspace.data_ptr(),
                                       _nbytes(workspace), _stream()),
           "sq_linear_fwd_contract")
    return out


def dgrad_workspace_bytes(m: int, p: W4Payload) -> int:
    return _lib.sq_linear_dgrad_workspace_bytes(m, p.abi())


def linear_dgrad(dy: torch.Tensor, p: W4Payload, out_dtype=torch.float32,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """sq_linear_dgrad: bf16 dy [M,N] -> dx = dy @ W_hat [M,K] (fp32 or bf16)."""
    _require(dy, torch.bfloat16, "dy")
    m = S.check_rows("dy", dy.shape, p.n)
    if out is None:
        out = torch.empty((m, p.k), dtype=out_dtype, device=dy.device)
    _require(out, out.dtype, "out")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, p.k):
        raise ValueError("out must be fp32 or bf16 of shape [M, K]")
    dt = SQ_BF16 if out.dtype == torch.bfloat16 else SQ_F32
    nbytes = dgrad_workspace_bytes(m, p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dy.device)
    _check(_lib.sq_linear_dgrad(dy.data_ptr(), m, p.abi(), out.data_ptr(), dt,
                                workspace.data_ptr(), _nbytes(workspace), _stream()),
           "sq_linear_dgrad")
    return out


def reconstruct_bf16(p: W4Payload, out: torch.Tensor | None = None):
    """sq_reconstruct_bf16: payload -> bf16 W_hat [N,K]."""
    if out is None:
        out = torch.empty((p.n, p.k), dtype=torch.bfloat16, device=p.codes.device)
    _require(out, torch.bfloat16, "out")
    S.check_out("out", out.shape, (p.n, p.k))
    _check(_lib.sq_reconstruct_bf16(p.abi(), out.data_ptr(), _stream()), "sq_reconstruct_bf16")
    return out


# ---------------------------------------------------------------- int8-residual mode
@dataclass
class W8Payload:
    """Device tensors of one int8-residual layer (layouts as in sq.h)."""
    codes: torch.Tensor      # int8 [N, K]
    scales: torch.Tensor     # float16 [N]
    up: torch.Tensor | None  # bfloat16 [N, rank]
    down: torch.Tensor | None  # bfloat16 [K, rank]

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1]

    @property
    def rank(self) -> int:
        return 0 if self.up is None else self.up.shape[1]

    def abi(self) -> SqW8:
        _require(self.codes, torch.int8, "codes")
        _require(self.scales, torch.float16, "scales")
        S.check_w8_payload(self.codes.shape, self.scales.shape, _shp(self.up), _shp(self.down))
        if self.up is not None:
            _require(self.up, torch.bfloat16, "up")
            _require(self.down, torch.bfloat16, "down")
        return SqW8(self.n, self.k, self.rank, 0, _ptr(self.codes), _ptr(self.scales),
                    _ptr(self.up), _ptr(self.down))


def empty_payload_w8(n: int, k: int, rank: int, device="cuda") -> W8Payload:
    up = torch.empty((n, rank), dtype=torch.bfloat16, device=device) if rank else None
    down = torch.empty((k, rank), dtype=torch.bfloat16, device=device) if rank else None
    return W8Payload(torch.empty((n, k), dtype=torch.int8, device=device),
                     torch.empty((n,), dtype=torch.float16, device=device), up, down)


def quantize_weight_w8(w: torch.Tensor, up: torch.Tensor | None, down: torch.Tensor | None,
                       want_fidx: bool = True, workspace: torch.Tensor | None = None):
    """sq_quantize_weight_w8: fp32 W [N,K] and bf16 factors -> (payload, fidx, flags tensor)."""
    _require(w, torch.float32, "w")
    n, k, rank = S.check_weight(w.shape, _shp(up), _shp(down), (16, 32, 64))
    p = empty_payload_w8(n, k, rank, w.device)
    p.up, p.down = up, down
    fidx = torch.empty((n,), dtype=torch.uint8, device=w.device) if want_fidx else None
    flags = torch.zeros(4, dtype=torch.int32, device=w.device)
    nbytes = _lib.sq_quantize_weight_w8_workspace_bytes(p.abi())
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    _check(_lib.sq_quantize_weight_w8(w.data_ptr(), p.abi(), _ptr(fidx), flags.data_ptr(),
                                      workspace.data_ptr(), _nbytes(workspace), _stream()),
           "sq_quantize_weight_w8")
    return p, fidx, flags


def reconstruct_bf16_w8(p: W8Payload, out: torch.Tensor | None = None):
    """sq_reconstruct_bf16_w8: int8-mode payload -> bf16 W_hat [N,K]."""
    if out is None:
        out = torch.empty((p.n, p.k), dtype=torch.bfloat16, device=p.codes.device)
    _require(out, torch.bfloat16, "out")
    S.check_out("out", out.shape, (p.n, p.k))
    _check(_lib.sq_reconstruct_bf16_w8(p.abi(), out.data_ptr(), _stream()),
           "sq_reconstruct_bf16_w8")
    return out


def fwd_w8_workspace_bytes(m: int, p: W8Payload) -> int:
    return _lib.sq_linear_fwd_w8_workspace_bytes(m, p.abi())


def linear_fwd_w8(x: torch.Tensor, p: W8Payload, out_dtype=torch.float32,
                  workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """sq_linear_fwd_w8: bf16 x [M,K] -> y [M,N] (fp32 or bf16) for an int8-mode payload."""
    _require(x, torch.bfloat16, "x")
    m = S.check_rows("x", x.shape, p.k)
    if out is None:
        out = torch.empty((m, p.n), dtype=out_dtype, device=x.device)
    _require(out, out.dtype, "out")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, p.n):
        raise ValueError("out must be fp32 or bf16 of shape [M, N]")
    dt = SQ_BF16 if out.dtype == torch.bfloat16 else SQ_F32
    nbytes = fwd_w8_workspace_bytes(m, p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check(_lib.sq_linear_fwd_w8(x.data_ptr(), m, p.abi(), out.data_ptr(), dt,
                                 workspace.data_ptr(), _nbytes(workspace), _stream()),
           "sq_linear_fwd_w8")
    return out


# ---------------------------------------------------------------- MXFP4 mode
@dataclass
class MX4Payload:
    """Device tensors of one MXFP4 layer (layouts as in sq.h)."""
    codes: torch.Tensor      # uint8 [N, K/2] E2M1 nibbles
    exps: torch.Tensor       # uint8 [N, K/32] E8M0 block exponents
    up: torch.Tensor | None  # bfloat16 [N, rank]
    down: torch.Tensor | None  # bfloat16 [K, rank]

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1] * 2

    @property
    def rank(self) -> int:
        return 0 if self.up is None else self.up.shape[1]

    def abi(self) -> SqMx4:
        _require(self.codes, torch.uint8, "codes")
        _require(self.exps, torch.uint8, "exps")
        S.check_mx4_payload(self.codes.shape, self.exps.shape, _shp(self.up), _shp(self.down))
        if self.up is not None:
            _require(self.up, torch.bfloat16, "up")
            _require(self.down, torch.bfloat16, "down")
        return SqMx4(self.n, self.k, self.rank, 0, _ptr(self.codes), _ptr(self.exps),
                     _ptr(self.up), _ptr(self.down))


def empty_payload_mx4(n: int, k: int, rank: int, device="cuda") -> MX4Payload:
    up = torch.empty((n, rank), dtype=torch.bfloat16, device=device) if rank else None
    down = torch.empty((k, rank), dtype=torch.bfloat16, device=device) if rank else None
    return MX4Payload(torch.empty((n, k // 2), dtype=torch.uint8, device=device),
                      torch.empty((n, k // 32), dtype=torch.uint8, device=device), up, down)


def quantize_weight_mx4(w: torch.Tensor, up: torch.Tensor | None, down: torch.Tensor | None):
    """sq_quantize_weight_mx4: fp32 W [N,K] and bf16 factors -> (payload, flags tensor)."""
    _require(w, torch.float32, "w")
    n, k, rank = S.check_weight(w.shape, _shp(up), _shp(down), (16, 32, 64))
    p = empty_payload_mx4(n, k, rank, w.device)
    p.up, p.down = up, down
    flags = torch.zeros(4, dtype=torch.int32, device=w.device)
    _check(_lib.sq_quantize_weight_mx4(w.data_ptr(), p.abi(), flags.data_ptr(), _stream()),
           "sq_quantize_weight_mx4")
    return p, flags


def quantize_act_mx4(x: torch.Tensor):
    """sq_quantize_act_mx4: bf16 x [M,K] -> (uint8 codes [M,K/2], uint8 exps [M,K/32]) of x @ H."""
    _require(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    xq = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    xs = torch.empty((m, k // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.sq_quantize_act_mx4(x.data_ptr(), m, k, xq.data_ptr(), xs.data_ptr(), _stream()),
           "sq_quantize_act_mx4")
    return xq, xs


def reconstruct_bf16_mx4(p: MX4Payload, out: torch.Tensor | None = None):
    """sq_reconstruct_bf16_mx4: MXFP4 payload -> bf16 W_hat [N,K]."""
    if out is None:
        out = torch.empty((p.n, p.k), dtype=torch.bfloat16, device=p.codes.device)
    _require(out, torch.bfloat16, "out")
    S.check_out("out", out.shape, (p.n, p.k))
    _check(_lib.sq_reconstruct_bf16_mx4(p.abi(), out.data_ptr(), _stream()),
           "sq_reconstruct_bf16_mx4")
    return out


def fwd_mx4_workspace_bytes(m: int, p: MX4Payload) -> int:
    return _lib.sq_linear_fwd_mx4_workspace_bytes(m, p.abi())


def linear_fwd_mx4(x: torch.Tensor, p: MX4Payload, out_dtype=torch.float32,
                   workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """sq_linear_fwd_mx4: bf16 x [M,K] -> y [M,N] (fp32 or bf16) for an MXFP4 payload."""
    _require(x, torch.bfloat16, "x")
    m = S.check_rows("x", x.shape, p.k)
    if out is None:
        out = torch.empty((m, p.n), dtype=out_dtype, device=x.device)
    _require(out, out.dtype, "out")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, p.n):
        raise ValueError("out must be fp32 or bf16 of shape [M, N]")
    dt = SQ_BF16 if out.dtype == torch.bfloat16 else SQ_F32
    nbytes = fwd_mx4_workspace_bytes(m, p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check(_lib.sq_linear_fwd_mx4(x.data_ptr(), m, p.abi(), out.data_ptr(), dt,
                                  workspace.data_ptr(), _nbytes(workspace), _stream()),
           "sq_linear_fwd_mx4")
    return out
