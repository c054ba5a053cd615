"""The streaming builder with its GPU steps: every quantized tensor of the slab
equals sq_quantize_weight on the stored factors, bit for bit, and matches the
CPU oracle's quantization of those factors under tie certification; a build
interrupted from the host resumes to the same bytes."""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401


def _source(path):
    from safetensors.torch import save_file
    g = torch.Generator().manual_seed(5)
    t = {"a.weight": torch.randn((256, 1024), generator=g) * 0.02,                 # host fp64 SVD
         "b.weight": (torch.randn((2048, 3072), generator=g) * 0.02).to(torch.bfloat16),  # randomized
         "b.bias": torch.randn((2048,), generator=g)}
    save_file(t, path)
    return t


def test_builder_matches_entry_point_and_resumes(tmp_path):
    import w4_gemm_amd as W
    from safetensors import safe_open
    from w4_gemm_amd import builder as B
    src = str(tmp_path / "m.safetensors")
    t = _source(src)
    out = B.build(src, str(tmp_path / "s1"), rank=32, group=32)
    d = torch.device("cuda")
    with safe_open(out, framework="pt") as f:
        assert torch.equal(f.get_tensor("b.bias"), t["b.bias"])
        for name in ("a.weight", "b.weight"):
            w = t[name].float().to(d)
            up, dn = f.get_tensor(f"{name}.lora_up").to(d), f.get_tensor(f"{name}.lora_down").to(d)
            p, fidx, flags = W.quantize_weight(w, up, dn, 32)
            torch.cuda.synchronize()
            assert int(flags[0]) == 0
            assert torch.equal(p.codes.cpu(), f.get_tensor(f"{name}.codes"))
            assert torch.equal(p.scales.cpu().view(torch.int16), f.get_tensor(f"{name}.scales").view(torch.int16))
            assert torch.equal(fidx.cpu(), f.get_tensor(f"{name}.fidx"))
            # and the oracle's quantization of the slab's own factors, tie-certified,
            # on sampled rows (the whole of the smaller weight)
            rows = np.arange(w.shape[0]) if w.shape[0] <= 256 else np.sort(
                np.random.default_rng(1).choice(w.shape[0], 256, replace=False))
            ups = O.bf16_decode(f.get_tensor(f"{name}.lora_up").view(torch.int16).numpy().view(np.uint16))
            dns = O.bf16_decode(f.get_tensor(f"{name}.lora_down").view(torch.int16).numpy().view(np.uint16))
            r = O.residual(t[name].float().numpy()[rows], ups[rows], dns)
            res = O.quantize_residual(r, 32)
            rep = O.check_device_quant(
                r, res, 32, O.unpack(f.get_tensor(f"{name}.codes").numpy()[rows]),
                f.get_tensor(f"{name}.scales").numpy()[rows].astype(np.float64),
                f.get_tensor(f"{name}.fidx").numpy()[rows])
            print(f"{name}: slab vs oracle {rep}")
            assert rep["ok"], rep
            # the slab reconstructs the weight to the codec's accuracy
            what = W.reconstruct_bf16(p).float()
            e = float((what - w).norm() / w.norm())
            print(f"{name}: relF(W_hat, W) = {e:.4f}")
            assert e < 0.15

    class Stop(Exception):
        pass

    def stop(name):
        if name == "b.weight":
            raise Stop()
    with pytest.raises(Stop):
        B.build(src, str(tmp_path / "s2"), rank=32, group=32, after_write=stop)
    out2 = B.build(src, str(tmp_path / "s2"), rank=32, group=32)
    assert open(out2, "rb").read() == open(out, "rb").read()


@pytest.mark.parametrize("fmt,rank", [("int8", 16), ("mxfp4", 32)])
def test_builder_other_codecs_match_entry_points(tmp_path, fmt, rank):
    import w4_gemm_amd as W
    from safetensors import safe_open
    from w4_gemm_amd import builder as B
    src = str(tmp_path / "m.safetensors")
    t = _source(src)
    out = B.build(src, str(tmp_path / fmt), rank=rank, group=32, fmt=fmt)
    d = torch.device("cuda")
    with safe_open(out, framework="pt") as f:
        assert f.metadata()["codec"] == fmt
        for name in ("a.weight", "b.weight"):
            w = t[name].float().to(d)
            up, dn = f.get_tensor(f"{name}.lora_up").to(d), f.get_tensor(f"{name}.lora_down").to(d)
            if fmt == "int8":
                p, fidx, flags = W.quantize_weight_w8(w, up, dn)
                torch.cuda.synchronize()
                assert torch.equal(p.codes.cpu(), f.get_tensor(f"{name}.codes"))
                assert torch.equal(p.scales.cpu().view(torch.int16), f.get_tensor(f"{name}.scales").view(torch.int16))
                assert torch.equal(fidx.cpu(), f.get_tensor(f"{name}.fidx"))
                what = W.reconstruct_bf16_w8(p).float()
            else:
                p, flags = W.quantize_weight_mx4(w, up, dn)
                torch.cuda.synchronize()
                assert torch.equal(p.codes.cpu(), f.get_tensor(f"{name}.codes"))
                assert torch.equal(p.exps.cpu(), f.get_tensor(f"{name}.exps"))
                what = W.reconstruct_bf16_mx4(p).float()
            assert int(flags[0]) == 0
            e = float((what - w).norm() / w.norm())
            print(f"{fmt} {name}: relF(W_hat, W) = {e:.4f}")
            assert e < 0.15
