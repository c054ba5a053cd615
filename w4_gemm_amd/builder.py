"""Streaming, restartable builder of a W4 slab from a safetensors checkpoint.

SquareQ README, "SquareQ v3 - W4": one artifact holds every quantized linear
layer ("One artifact" bullet), and the builder streams the source and, killed
mid-build, resumes to byte-identical output ("Builder (streaming,
restartable)" paragraph).  This is that builder over libsq: per linear weight
the rank-r split runs first (host fp64 SVD, or a seeded randomized SVD on the
GPU for large weights), then sq_quantize_weight on the GPU.

Plan (a pure function of the source header and the options):
  source tensors in name order; a 2-D floating tensor [N, K] with K % 256 == 0
  whose name matches `include` becomes, with the default W4 codec,
      <name>.codes      U8    [N, K/2]
      <name>.scales     F16   [N, K/group]
      <name>.fidx       U8    [N, K/group]   (chosen fraction index)
      <name>.lora_up    BF16  [N, rank]      (rank > 0)
      <name>.lora_down  BF16  [K, rank]      (rank > 0)
  and every other tensor is copied byte for byte.  The other codecs of the
  library (the page's v3.1 int8-residual mode and the FP4 alternative of its
  "Residual codecs" bullet, as MXFP4) replace the first three by
      int8:  <name>.codes I8 [N, K], <name>.scales F16 [N], <name>.fidx U8 [N]
      mxfp4: <name>.codes U8 [N, K/2] (E2M1 nibbles), <name>.exps U8 [N, K/32]  The output is a
  safetensors file: header (padded with spaces to a multiple of 8 bytes),
  then the data regions in plan order, contiguous.

Restart protocol (`<out_dir>/slab.safetensors.partial` during the build,
`<out_dir>/build_state.json` beside it):
  1. the partial file is created once at its final size (header + zeros);
  2. each source tensor not yet recorded is converted, its bytes are written
     at their offsets and the file is fsync'ed; only then is the tensor
     recorded (with the sha256 of its bytes) in the state file, which is
     replaced atomically (temporary file, fsync, rename);
  3. when every tensor is recorded the partial file is renamed to
     slab.safetensors and the state is marked complete.
A kill at any point loses at most the tensor in progress; its region is
rewritten on the next run.  Every tensor's bytes are a deterministic function
of the source bytes and the options, so a resumed build is byte-identical to
an uninterrupted one.  The state file also records the source's size and the
sha256 of every source tensor's bytes: a resume against a source whose
contents changed (even with an identical header) is refused, and every
recorded tensor's output region is re-hashed against its recorded sha256
before it is trusted (a mismatch is rebuilt).  Peak host memory is about one
source tensor and its outputs.

Usage: python -m w4_gemm_amd.builder --src model.safetensors --out-dir slab \
           [--format w4|int8|mxfp4] [--rank 32] [--group 32] [--svd auto|exact|randomized]
           [--include REGEX]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import mmap
import os
import re
import struct
import sys
import time
import zlib
from dataclasses import dataclass, field

import numpy as np

FORMAT = "squareq-v3-w4"
SLAB = "slab.safetensors"
PARTIAL = SLAB + ".partial"
STATE = "build_state.json"
ITEMSIZE = {"F32": 4, "F16": 2, "BF16": 2, "U8": 1, "I8": 1, "F64": 8, "I32": 4, "I64": 8,
            "U16": 2, "I16": 2, "BOOL": 1}
FLOAT_IN = ("F32", "F16", "BF16")
EXACT_SVD_MAX = 1 << 22   # weights with at most this many elements get the host fp64 SVD
RSVD_OVERSAMPLE = 96      # randomized split: extra sample columns beyond the rank
RSVD_ITERS = 16           # randomized split: power iterations


# ---------------------------------------------------------------- safetensors header
def read_header(path: str):
    """(header dict without __metadata__, metadata, data start offset) of a safetensors file."""
    with open(path, "rb") as f:
        (n,) = struct.unpack("<Q", f.read(8))
        hdr = json.loads(f.read(n))
    meta = hdr.pop("__metadata__", {}) or {}
    return hdr, meta, 8 + n


@dataclass
class OutTensor:
    name: str
    dtype: str
    shape: tuple
    offset: int = 0   # relative to the data start

    @property
    def nbytes(self) -> int:
        return int(np.prod(self.shape, dtype=np.int64)) * ITEMSIZE[self.dtype]


@dataclass
class Unit:
    """One source tensor and the output tensors made from it."""
    src: str
    kind: str                       # "w4" or "copy"
    src_dtype: str
    src_shape: tuple
    src_range: tuple                # byte range in the source data section
    outs: list = field(default_factory=list)


@dataclass
class Plan:
    units: list
    header_bytes: bytes
    data_start: int
    total: int
    digest: str


CODECS = ("w4", "int8", "mxfp4")


def codec_outputs(fmt: str, name: str, n: int, k: int, group: int):
    """The quantizer's output tensors of one weight, in file order."""
    if fmt == "int8":
        return [OutTensor(f"{name}.codes", "I8", (n, k)), OutTensor(f"{name}.scales", "F16", (n,)),
                OutTensor(f"{name}.fidx", "U8", (n,))]
    if fmt == "mxfp4":
        return [OutTensor(f"{name}.codes", "U8", (n, k // 2)),
                OutTensor(f"{name}.exps", "U8", (n, k // 32))]
    return [OutTensor(f"{name}.codes", "U8", (n, k // 2)),
            OutTensor(f"{name}.scales", "F16", (n, k // group)),
            OutTensor(f"{name}.fidx", "U8", (n, k // group))]


def make_plan(src: str, rank: int, group: int, svd: str, include: str, fmt: str = "w4") -> Plan:
    hdr, meta, _ = read_header(src)
    pat = re.compile(include)
    units = []
    for name in sorted(hdr):
        t = hdr[name]
        dt, shape, rng = t["dtype"], tuple(t["shape"]), tuple(t["data_offsets"])
        quant = (dt in FLOAT_IN and len(shape) == 2 and shape[1] % 256 == 0 and shape[1] >= 256
                 and shape[0] >= 1 and pat.search(name) is not None)
        u = Unit(name, "w4" if quant else "copy", dt, shape, rng)
        if quant:
            n, k = shape
            u.outs = codec_outputs(fmt, name, n, k, group)
            if rank > 0:
                u.outs += [OutTensor(f"{name}.lora_up", "BF16", (n, rank)),
                           OutTensor(f"{name}.lora_down", "BF16", (k, rank))]
        else:
            u.outs = [OutTensor(name, dt, shape)]
        units.append(u)
    off = 0
    entries = {"__metadata__": {"format": FORMAT, "rank": str(rank), "group": str(group),
                                "svd": svd, "include": include}}
    if fmt != "w4":
        entries["__metadata__"]["codec"] = fmt
    for u in units:
        for o in u.outs:
            o.offset = off
            off += o.nbytes
            entries[o.name] = {"dtype": o.dtype, "shape": list(o.shape),
                               "data_offsets": [o.offset, o.offset + o.nbytes]}
    js = json.dumps(entries, separators=(",", ":")).encode()
    js += b" " * (-(8 + len(js)) % 8)
    header = struct.pack("<Q", len(js)) + js
    digest = hashlib.sha256(header + json.dumps(
        [(u.src, u.src_dtype, list(u.src_shape)) for u in units]).encode()).hexdigest()
    return Plan(units, header, len(header), off, digest)


# ---------------------------------------------------------------- per-tensor steps (GPU)
def _to_f32(raw: memoryview, dtype: str, shape) -> np.ndarray:
    if dtype == "F32":
        a = np.frombuffer(raw, dtype=np.float32).copy()   # no view into the source map
    elif dtype == "F16":
        a = np.frombuffer(raw, dtype=np.float16).astype(np.float32)
    else:   # BF16: the high half of an fp32
        a = (np.frombuffer(raw, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return a.reshape(shape)


def gpu_lowrank(w: np.ndarray, rank: int, name: str, svd: str):
    """bf16 bit patterns (up [N,r], down [K,r]) of the rank-r split U sqrt(S), V sqrt(S).

    exact: host fp64 LAPACK SVD, one rounding to bf16.  randomized: a seeded
    randomized SVD on the GPU in fp64 (r + RSVD_OVERSAMPLE sample columns,
    RSVD_ITERS power iterations, seed from the tensor name), for weights too
    large for the host SVD.  Its rank-r residual energy stays within 1e-4 of
    the Eckart-Young optimum on the layer distributions (pinned on the CPU);
    the residual absorbs any difference from the exact factors.
    """
    import torch
    if svd == "auto":
        svd = "exact" if w.size <= EXACT_SVD_MAX else "randomized"
    if svd == "exact":
        from .svd_init import svd_init
        up, dn = svd_init(w, rank)
        return (up.view(torch.int16).numpy().view(np.uint16), dn.view(torch.int16).numpy().view(np.uint16))
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(name.encode()))
    wd = torch.from_numpy(w).cuda().double()
    u, s, v = randomized_split(torch, wd, rank, g)
    r = s[:rank].sqrt()
    from .svd_init import _bf16_from_f64      # one rounding from fp64, as the exact split
    up = _bf16_from_f64((u[:, :rank] * r).cpu().numpy())
    dn = _bf16_from_f64((v[:, :rank] * r).cpu().numpy())
    return up.view(torch.int16).numpy().view(np.uint16), dn.view(torch.int16).numpy().view(np.uint16)


def randomized_split(torch, a, rank: int, gen):
    """Top singular triplets of `a` by the randomized range finder below."""
    return _svd_lowrank(torch, a, min(rank + RSVD_OVERSAMPLE, min(a.shape)), gen, RSVD_ITERS)


def _svd_lowrank(torch, a, q, gen, niter=2):
    """Randomized range finder + small SVD (Halko et al. 2011, algorithm 4.4)."""
    m, n = a.shape
    omega = torch.randn((n, q), generator=gen, device=a.device, dtype=a.dtype)
    y = a @ omega
    qm, _ = torch.linalg.qr(y)
    for _ in range(niter):
        z, _ = torch.linalg.qr(a.T @ qm)
        qm, _ = torch.linalg.qr(a @ z)
    b = qm.T @ a
    ub, s, vh = torch.linalg.svd(b, full_matrices=False)
    return qm @ ub, s, vh.T


def gpu_quantize(w: np.ndarray, up_bits, dn_bits, group: int):
    """sq_quantize_weight on the GPU: (codes u8, scale bits u16, fidx u8) as host arrays."""
    import torch
    from . import api
    d = torch.device("cuda")
    bf = (lambda b: None if b is None else
          torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(d))
    p, fidx, flags = api.quantize_weight(torch.from_numpy(np.ascontiguousarray(w)).to(d),
                                         bf(up_bits), bf(dn_bits), group)
    torch.cuda.synchronize()
    f = int(flags[0])
    if f:
        raise FloatingPointError(f"quantizer flags {f:#x} (1 non-finite weight, 2 fp16 scale overflow)")
    return (p.codes.cpu().numpy(), p.scales.view(torch.int16).cpu().numpy().view(np.uint16),
            fidx.cpu().numpy())


def gpu_quantize_w8(w: np.ndarray, up_bits, dn_bits, group: int):
    """sq_quantize_weight_w8 on the GPU: (codes i8, scale bits u16 [N], fidx u8 [N])."""
    import torch
    from . import api
    d = torch.device("cuda")
    bf = (lambda b: None if b is None else
          torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(d))
    p, fidx, flags = api.quantize_weight_w8(torch.from_numpy(np.ascontiguousarray(w)).to(d),
                                            bf(up_bits), bf(dn_bits))
    torch.cuda.synchronize()
    f = int(flags[0])
    if f:
        raise FloatingPointError(f"quantizer flags {f:#x} (1 non-finite weight, 2 fp16 scale overflow)")
    return (p.codes.cpu().numpy(), p.scales.view(torch.int16).cpu().numpy().view(np.uint16),
            fidx.cpu().numpy())


def gpu_quantize_mx(w: np.ndarray, up_bits, dn_bits, group: int):
    """sq_quantize_weight_mx4 on the GPU: (codes u8 [N, K/2], exps u8 [N, K/32])."""
    import torch
    from . import api
    d = torch.device("cuda")
    bf = (lambda b: None if b is None else
          torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(d))
    p, flags = api.quantize_weight_mx4(torch.from_numpy(np.ascontiguousarray(w)).to(d),
                                       bf(up_bits), bf(dn_bits))
    torch.cuda.synchronize()
    if int(flags[0]):
        raise FloatingPointError(f"quantizer flags {int(flags[0]):#x} (1 non-finite residual)")
    return p.codes.cpu().numpy(), p.exps.cpu().numpy()


GPU_QUANTIZE = {"w4": gpu_quantize, "int8": gpu_quantize_w8, "mxfp4": gpu_quantize_mx}


# ---------------------------------------------------------------- the build
def source_digest(src: str) -> str:
    """sha256 over the source's size and the sha256 of each tensor's bytes, in name order."""
    hdr, _, start = read_header(src)
    h = hashlib.sha256(str(os.path.getsize(src)).encode())
    with open(src, "rb") as f, mmap.mmap(f.fileno(), 0, access=mmap.ACCESS_READ) as m:
        for name in sorted(hdr):
            a, b = hdr[name]["data_offsets"]
            h.update(name.encode() + b"\0" + hashlib.sha256(m[start + a:start + b]).digest())
    return h.hexdigest()


def _region_sha(fd: int, plan: Plan, unit: Unit) -> str:
    h = hashlib.sha256()
    for o in unit.outs:
        h.update(os.pread(fd, o.nbytes, plan.data_start + o.offset))
    return h.hexdigest()


def _write_state(out_dir: str, state: dict):
    tmp = os.path.join(out_dir, STATE + ".tmp")
    with open(tmp, "w") as f:
        json.dump(state, f, indent=1, sort_keys=True)
        f.flush()
        os.fsync(f.fileno())
    os.replace(tmp, os.path.join(out_dir, STATE))
    dfd = os.open(out_dir, os.O_RDONLY)
    try:
        os.fsync(dfd)
    finally:
        os.close(dfd)


def build(src: str, out_dir: str, rank: int = 32, group: int = 32, svd: str = "auto",
          include: str = ".*", quantize=None, lowrank=None, after_write=None, log=None,
          fmt: str = "w4") -> str:
    """Build (or resume) the slab; returns the path of the finished file.

    quantize(w_f32, up_bits, down_bits, group) -> the codec's arrays in file
    order (W4: codes, scale_bits, fidx) and lowrank(w_f32, rank, name) ->
    (up_bits, down_bits) default to the GPU steps above.  after_write(unit_name)
    is called once a tensor's first output is written and before the rest (a
    hook for interruption tests).
    """
    if fmt not in CODECS:
        raise ValueError(f"format must be one of {CODECS}")
    ranks = (0, 32, 64) if fmt == "w4" else (0, 16, 32, 64)
    if group not in (32, 64) or rank not in ranks:
        raise ValueError(f"group must be 32 or 64 and rank one of {ranks}")
    if svd not in ("auto", "exact", "randomized"):
        raise ValueError("svd must be auto, exact or randomized")
    quantize = quantize or GPU_QUANTIZE[fmt]
    lowrank = lowrank or (lambda w, r, name: gpu_lowrank(w, r, name, svd))
    os.makedirs(out_dir, exist_ok=True)
    plan = make_plan(src, rank, group, svd, include, fmt)
    final, partial = os.path.join(out_dir, SLAB), os.path.join(out_dir, PARTIAL)
    spath = os.path.join(out_dir, STATE)
    sdig = source_digest(src)
    state = None
    if os.path.exists(spath):
        with open(spath) as f:
            state = json.load(f)
        if state.get("plan") != plan.digest or state.get("source") != sdig:
            raise RuntimeError(f"{out_dir} holds a build of different inputs or options; "
                               "remove it or choose another directory")
        if state.get("complete") and os.path.exists(final):
            return final
    if state is None or not os.path.exists(partial):
        with open(partial, "wb") as f:
            f.write(plan.header_bytes)
            f.truncate(plan.data_start + plan.total)
            f.flush()
            os.fsync(f.fileno())
        state = {"plan": plan.digest, "source": sdig, "done": {}, "complete": False}
        _write_state(out_dir, state)
    else:
        # trust a recorded tensor only if its bytes on disk still hash to the record
        fd = os.open(partial, os.O_RDONLY)
        try:
            stale = [u.src for u in plan.units
                     if u.src in state["done"] and _region_sha(fd, plan, u) != state["done"][u.src]]
        finally:
            os.close(fd)
        for name in stale:
            del state["done"][name]
        if stale:
            _write_state(out_dir, state)
    _, _, src_start = read_header(src)
    t0 = time.time()
    with open(src, "rb") as sf, mmap.mmap(sf.fileno(), 0, access=mmap.ACCESS_READ) as sm:
        fd = os.open(partial, os.O_RDWR)
        try:
            for u in plan.units:
                if u.src in state["done"]:
                    continue
                raw = memoryview(sm)[src_start + u.src_range[0]:src_start + u.src_range[1]]
                if u.kind == "copy":
                    blobs = [bytes(raw)]
                else:
                    w = _to_f32(raw, u.src_dtype, u.src_shape)
                    up = dn = None
                    if rank > 0:
                        up, dn = lowrank(w, rank, u.src)
                    blobs = [np.ascontiguousarray(a).tobytes() for a in quantize(w, up, dn, group)]
                    if rank > 0:
                        blobs += [np.ascontiguousarray(up, np.uint16).tobytes(),
                                  np.ascontiguousarray(dn, np.uint16).tobytes()]
                    del w
                del raw
                h = hashlib.sha256()
                for i, (o, b) in enumerate(zip(u.outs, blobs)):
                    if len(b) != o.nbytes:
                        raise RuntimeError(f"{o.name}: {len(b)} bytes, plan says {o.nbytes}")
                    os.pwrite(fd, b, plan.data_start + o.offset)
                    h.update(b)
                    if i == 0 and after_write:
                        after_write(u.src)      # part of the tensor is on disk, none recorded
                os.fsync(fd)
                state["done"][u.src] = h.hexdigest()
                _write_state(out_dir, state)
                if log:
                    log(f"{u.src}: {u.kind} {u.src_shape} done ({time.time() - t0:.1f} s)")
        finally:
            os.close(fd)
    os.replace(partial, final)
    state["complete"] = True
    _write_state(out_dir, state)
    return final


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--src", required=True)
    ap.add_argument("--out-dir", required=True)
    ap.add_argument("--rank", type=int, default=32)
    ap.add_argument("--group", type=int, default=32)
    ap.add_argument("--svd", default="auto", choices=("auto", "exact", "randomized"))
    ap.add_argument("--include", default=".*")
    ap.add_argument("--format", default="w4", choices=CODECS)
    a = ap.parse_args(argv)
    path = build(a.src, a.out_dir, a.rank, a.group, a.svd, a.include,
                 log=lambda s: print(s, flush=True), fmt=a.format)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
