"""The streaming builder's plan, file format and restart protocol, on the CPU.

The per-tensor steps are the oracle's (SVD split and quantizer, injected in
place of the GPU ones), so these tests need no GPU; the GPU steps themselves
are checked against the device entry points in test_gpu_builder.py.
"""
import json
import os
import signal
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle as O
from w4_gemm_amd import builder as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def oracle_lowrank(w, rank, name):
    up, dn = O.svd_init(np.asarray(w, np.float64), rank)
    bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits(up), bits(dn)


def oracle_quantize(w, up_bits, dn_bits, group):
    dec = lambda b: (np.zeros((w.shape[0] if b is up_bits else w.shape[1], 0)) if b is None
                     else O.bf16_decode(b))
    res = O.quantize_weight(np.asarray(w, np.float64), dec(up_bits), dec(dn_bits), group)
    return O.pack(res.q), res.scale.astype(np.float16).view(np.uint16), res.fidx


def make_source(path, seed=0):
    from safetensors.torch import save_file
    g = torch.Generator().manual_seed(seed)
    t = {
        "blocks.0.attn.q.weight": torch.randn((48, 512), generator=g) * 0.05,
        "blocks.0.attn.q.bias": torch.randn((48,), generator=g),
        "blocks.0.mlp.up.weight": (torch.randn((40, 768), generator=g) * 0.05).to(torch.bfloat16),
        "blocks.0.norm.weight": torch.ones((512,)),
        "embed.weight": torch.randn((10, 100), generator=g),          # K % 256 != 0: copied
        "blocks.1.mlp.down.weight": (torch.randn((32, 256), generator=g) * 0.05).to(torch.float16),
    }
    save_file(t, path)
    return t


def build(src, out, **kw):
    return B.build(src, out, rank=32, group=32, svd="exact", quantize=oracle_quantize,
                   lowrank=oracle_lowrank, **kw)


@pytest.fixture()
def src(tmp_path):
    p = str(tmp_path / "model.safetensors")
    return p, make_source(p)


def test_plan_layout(src):
    path, t = src
    plan = B.make_plan(path, 32, 32, "exact", ".*")
    kinds = {u.src: u.kind for u in plan.units}
    assert kinds["blocks.0.attn.q.weight"] == "w4" and kinds["blocks.0.mlp.up.weight"] == "w4"
    assert kinds["blocks.1.mlp.down.weight"] == "w4"
    assert kinds["embed.weight"] == "copy" and kinds["blocks.0.norm.weight"] == "copy"
    offs = sorted((o.offset, o.nbytes) for u in plan.units for o in u.outs)
    pos = 0
    for off, nb in offs:                     # contiguous, no holes
        assert off == pos
        pos += nb
    assert pos == plan.total and plan.data_start % 8 == 0
    assert B.make_plan(path, 32, 32, "exact", ".*").header_bytes == plan.header_bytes
    assert B.make_plan(path, 32, 64, "exact", ".*").digest != plan.digest
    only = B.make_plan(path, 32, 32, "exact", r"mlp\.up")
    assert [u.src for u in only.units if u.kind == "w4"] == ["blocks.0.mlp.up.weight"]


def test_build_contents(src, tmp_path):
    path, t = src
    out = build(path, str(tmp_path / "slab"))
    from safetensors import safe_open
    with safe_open(out, framework="pt") as f:
        assert f.metadata()["format"] == B.FORMAT
        keys = set(f.keys())
        for name in ("blocks.0.attn.q.bias", "blocks.0.norm.weight", "embed.weight"):
            assert torch.equal(f.get_tensor(name), t[name])
        for name in ("blocks.0.attn.q.weight", "blocks.0.mlp.up.weight", "blocks.1.mlp.down.weight"):
            w = t[name].float().numpy()
            up_b, dn_b = oracle_lowrank(w, 32, name)
            codes, sb, fidx = oracle_quantize(w, up_b, dn_b, 32)
            assert {f"{name}.{s}" for s in ("codes", "scales", "fidx", "lora_up", "lora_down")} <= keys
            assert np.array_equal(f.get_tensor(f"{name}.codes").numpy(), codes)
            assert np.array_equal(f.get_tensor(f"{name}.scales").view(torch.int16).numpy().view(np.uint16), sb)
            assert np.array_equal(f.get_tensor(f"{name}.fidx").numpy(), fidx)
            assert np.array_equal(f.get_tensor(f"{name}.lora_up").view(torch.int16).numpy().view(np.uint16), up_b)
            assert f.get_tensor(f"{name}.lora_down").shape == (w.shape[1], 32)
    state = json.load(open(tmp_path / "slab" / B.STATE))
    assert state["complete"] and len(state["done"]) == 6
    # a finished build is left alone
    before = open(out, "rb").read()
    assert build(path, str(tmp_path / "slab")) == out and open(out, "rb").read() == before
    # a different plan in the same directory is refused
    with pytest.raises(RuntimeError):
        B.build(path, str(tmp_path / "slab"), rank=32, group=64, svd="exact",
                quantize=oracle_quantize, lowrank=oracle_lowrank)


CHILD = r"""
import os, signal, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, os.path.join({root!r}, "tests")); sys.path.insert(0, os.path.join({root!r}, "oracle"))
from test_builder_cpu import build
def die(name):
    if name == {victim!r}:
        os.kill(os.getpid(), signal.SIGKILL)
build({src!r}, {out!r}, after_write=die)
"""


@pytest.mark.parametrize("victim", ["blocks.0.mlp.up.weight", "blocks.1.mlp.down.weight",
                                    "embed.weight"])
def test_kill_and_resume_is_byte_identical(src, tmp_path, victim):
    path, _ = src
    ref = build(path, str(tmp_path / "ref"))
    out = str(tmp_path / "killed")
    code = CHILD.format(root=ROOT, victim=victim, src=path, out=out)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == -signal.SIGKILL, r.stderr
    state = json.load(open(os.path.join(out, B.STATE)))
    assert not state["complete"] and victim not in state["done"]
    assert os.path.exists(os.path.join(out, B.PARTIAL)) and not os.path.exists(os.path.join(out, B.SLAB))
    done_before = set(state["done"])
    seen = []
    final = build(path, out, after_write=seen.append)
    assert set(seen).isdisjoint(done_before) and victim in seen     # only the rest is redone
    assert open(final, "rb").read() == open(ref, "rb").read()


def oracle_quantize_w8(w, up_bits, dn_bits, group):
    dec = lambda b: (np.zeros((w.shape[0] if b is up_bits else w.shape[1], 0)) if b is None
                     else O.bf16_decode(b))
    res = O.quantize_weight_w8(np.asarray(w, np.float64), dec(up_bits), dec(dn_bits))
    return res.q.astype(np.int8), res.scale.astype(np.float16).view(np.uint16), res.fidx


def oracle_quantize_mx(w, up_bits, dn_bits, group):
    dec = lambda b: (np.zeros((w.shape[0] if b is up_bits else w.shape[1], 0)) if b is None
                     else O.bf16_decode(b))
    codes, exps = O.quantize_weight_mx(np.asarray(w, np.float64), dec(up_bits), dec(dn_bits))
    return O.mx_pack(codes), exps


@pytest.mark.parametrize("fmt,rank", [("int8", 16), ("mxfp4", 32)])
def test_build_other_codecs(src, tmp_path, fmt, rank):
    path, t = src
    q = oracle_quantize_w8 if fmt == "int8" else oracle_quantize_mx
    out = B.build(path, str(tmp_path / fmt), rank=rank, group=32, svd="exact", quantize=q,
                  lowrank=oracle_lowrank, fmt=fmt)
    from safetensors import safe_open
    with safe_open(out, framework="pt") as f:
        assert f.metadata()["codec"] == fmt
        assert torch.equal(f.get_tensor("embed.weight"), t["embed.weight"])
        for name in ("blocks.0.attn.q.weight", "blocks.1.mlp.down.weight"):
            w = t[name].float().numpy()
            up_b, dn_b = oracle_lowrank(w, rank, name)
            arrays = q(w, up_b, dn_b, 32)
            names = ("codes", "scales", "fidx") if fmt == "int8" else ("codes", "exps")
            for s, a in zip(names, arrays):
                got = f.get_tensor(f"{name}.{s}")
                got = got.view(torch.int16).numpy().view(np.uint16) if got.dtype == torch.float16 else got.numpy()
                assert np.array_equal(got, a), (name, s)
            assert f.get_tensor(f"{name}.lora_up").shape == (w.shape[0], rank)
    with pytest.raises(ValueError):
        B.build(path, str(tmp_path / "bad"), rank=16, group=32, fmt="w4")


class _Stop(Exception):
    pass


def _partial_build(path, out, victim):
    """Run a build that stops (in process) once `victim`'s first output is written."""
    def stop(name):
        if name == victim:
            raise _Stop()
    with pytest.raises(_Stop):
        build(path, out, after_write=stop)


def test_resume_refuses_changed_source(src, tmp_path):
    path, t = src
    out = str(tmp_path / "slab")
    _partial_build(path, out, "blocks.1.mlp.down.weight")
    # same header, different bytes of one tensor
    t2 = dict(t)
    t2["blocks.0.attn.q.weight"] = t["blocks.0.attn.q.weight"] * 2
    from safetensors.torch import save_file
    save_file(t2, path)
    assert B.make_plan(path, 32, 32, "exact", ".*").digest == \
        B.make_plan(path, 32, 32, "exact", ".*").digest
    with pytest.raises(RuntimeError):
        build(path, out)


def test_resume_rebuilds_a_corrupted_region(src, tmp_path):
    path, _ = src
    ref = build(path, str(tmp_path / "ref"))
    out = str(tmp_path / "slab")
    _partial_build(path, out, "blocks.1.mlp.down.weight")
    state = json.load(open(os.path.join(out, B.STATE)))
    plan = B.make_plan(path, 32, 32, "exact", ".*")
    victim = next(u for u in plan.units if u.src in state["done"] and u.kind == "w4")
    with open(os.path.join(out, B.PARTIAL), "r+b") as f:
        f.seek(plan.data_start + victim.outs[-1].offset + 3)   # a byte of its lora_down
        b = f.read(1)
        f.seek(-1, 1)
        f.write(bytes([b[0] ^ 0x40]))
    seen = []
    final = build(path, out, after_write=seen.append)
    assert victim.src in seen                                   # rebuilt, not trusted
    assert open(final, "rb").read() == open(ref, "rb").read()
