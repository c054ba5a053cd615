"""Host-side steps of the package that need no GPU.

* the product's rank-r SVD split (w4_gemm_amd.svd_init) against the oracle's
  (the "Low-rank branch" bullet of the SquareQ README's "SquareQ v3 - W4"
  section: a rank-32 SVD of the weight, stored in bf16), bit for bit;
* the randomized split the builder uses for large weights, against the
  Eckart-Young optimum of the exact SVD;
* the wrappers' shape checks, which stand between torch tensors and the raw
  pointers of the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen_weight
from w4_gemm_amd import shapes as S
from w4_gemm_amd import builder as B
from w4_gemm_amd.svd_init import svd_init


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n,k,rank,spike", [(64, 512, 32, 4), (96, 256, 16, 8), (512, 256, 32, 8),
                                            (300, 768, 64, 8), (1024, 1024, 32, 8)])
def test_svd_init_matches_oracle(n, k, rank, spike):
    rng = np.random.default_rng(n + k + rank)
    w = gen_weight(rng, n, k, spike)
    up, dn = svd_init(w, rank)
    oup, odn = O.svd_init(w, rank)
    # the oracle holds bf16 values in fp64; the product returns bf16 tensors
    assert np.array_equal(_bits(up), (oup.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    assert np.array_equal(_bits(dn), (odn.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    assert np.array_equal(up.double().numpy() @ dn.double().numpy().T, oup @ odn.T)


def test_svd_init_rank0_and_torch_input():
    w = gen_weight(np.random.default_rng(3), 32, 256, 4)
    assert svd_init(w, 0) == (None, None)
    a, b = svd_init(torch.from_numpy(w), 32)
    c, d = svd_init(w, 32)
    assert torch.equal(a, c) and torch.equal(b, d)


def test_bf16_rounding_of_split_is_single():
    # values exactly halfway between two bf16 numbers after fp32 rounding but
    # not before: one rounding from fp64 keeps them on the correct side
    from w4_gemm_amd.svd_init import _bf16_from_f64
    base = 1.0 + 2.0 ** -8                       # halfway between bf16 1 and 1+2^-7
    v = np.array([base + 2.0 ** -40, base - 2.0 ** -40, -(base + 2.0 ** -40), base])
    got = _bits(_bf16_from_f64(v))
    want = (O.bf16_round(v).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got, want)
    assert got[0] != got[1]


@pytest.mark.parametrize("n,k", [(4096, 1536), (1536, 4096)])
def test_randomized_split_near_eckart_young(n, k):
    rng = np.random.default_rng(7)
    w = gen_weight(rng, n, k, 8).astype(np.float64)
    s = np.linalg.svd(w, compute_uv=False)
    for seed in (0, 1):
        u, sv, v = B.randomized_split(torch, torch.from_numpy(w), 32, torch.Generator().manual_seed(seed))
        u, sv, v = u[:, :32].numpy(), sv[:32].numpy(), v[:, :32].numpy()
        resid = ((w - (u * sv) @ v.T) ** 2).sum()
        opt = (s[32:] ** 2).sum()                  # Eckart-Young: the best rank-32 residual
        assert opt <= resid <= opt * (1 + 1e-4)
        assert np.abs(sv / s[:32] - 1).max() < 2e-3
        assert np.allclose(u.T @ u, np.eye(32), atol=1e-10)   # orthonormal factors


def test_randomized_split_is_deterministic():
    w = torch.from_numpy(gen_weight(np.random.default_rng(9), 600, 512, 8).astype(np.float64))
    a = B.randomized_split(torch, w, 32, torch.Generator().manual_seed(5))
    b = B.randomized_split(torch, w, 32, torch.Generator().manual_seed(5))
    assert all(torch.equal(x, y) for x, y in zip(a, b))


# ------------------------------------------------------------------ shape checks
def test_w4_payload_shapes():
    assert S.check_w4_payload((8, 256), (8, 16), (8, 32), (512, 32), 32) == (8, 512, 32)
    assert S.check_w4_payload((8, 256), (8, 8), None, None, 64) == (8, 512, 0)
    bad = [
        ((8, 256), (8, 8), (8, 32), (512, 32), 32),      # scales for group 64 with group 32
        ((8, 256), (8, 16), (8, 32), (256, 32), 32),     # down rows != K
        ((8, 256), (8, 16), (9, 32), (512, 32), 32),     # up rows != N
        ((8, 256), (8, 16), (8, 32), (512, 64), 32),     # ranks differ
        ((8, 256), (8, 16), (8, 16), (512, 16), 32),     # rank 16 is not a W4 rank
        ((8, 256), (8, 16), (8, 32), None, 32),          # one factor missing
        ((8, 100), (8, 6), None, None, 32),              # K not a multiple of 256
        ((8, 256), (8, 16), None, None, 16),             # group 16
        ((0, 256), (0, 16), None, None, 32),             # N = 0
        ((8,), (8, 16), None, None, 32),                 # codes not 2-D
    ]
    for args in bad:
        with pytest.raises(ValueError):
            S.check_w4_payload(*args)


def test_w8_and_mx4_payload_shapes():
    assert S.check_w8_payload((4, 512), (4,), (4, 16), (512, 16)) == (4, 512, 16)
    for args in [((4, 512), (4, 1), None, None), ((4, 500), (4,), None, None),
                 ((4, 512), (4,), (4, 16), (512, 32))]:
        with pytest.raises(ValueError):
            S.check_w8_payload(*args)
    assert S.check_mx4_payload((4, 256), (4, 16), None, None) == (4, 512, 0)
    for args in [((4, 256), (4, 8), None, None), ((4, 256), (4, 16), (4, 32), (256, 32))]:
        with pytest.raises(ValueError):
            S.check_mx4_payload(*args)


def test_operand_shapes():
    assert S.check_rows("x", (7, 512), 512) == 7
    assert S.check_rows("x", (0, 512), 512) == 0
    for shp in [(7, 256), (512,), (2, 7, 512)]:
        with pytest.raises(ValueError):
            S.check_rows("x", shp, 512)
    S.check_out("out", (3, 4), (3, 4))
    with pytest.raises(ValueError):
        S.check_out("out", (4, 3), (3, 4))
    assert S.check_weight((16, 512), (16, 32), (512, 32)) == (16, 512, 32)
    with pytest.raises(ValueError):
        S.check_weight((16, 512), (16, 16), (512, 16))            # W4 rank 16
    assert S.check_weight((16, 512), (16, 16), (512, 16), (16, 32, 64)) == (16, 512, 16)
    with pytest.raises(ValueError):
        S.check_weight((16, 300), None, None)
