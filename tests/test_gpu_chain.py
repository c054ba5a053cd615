"""The whole device chain on the layer shapes: W -> sq_quantize_weight ->
sq_linear_fwd / sq_reconstruct_bf16, against the CPU oracle on sampled rows.

For each of the four full-size shapes (SquareQ README, "SquareQ v3 - W4": the
shapes of its NVFP4-vs-bf16 table) the weight of the seeded recipe is
quantized on the GPU; then
  * sampled rows of the device payload are checked against the oracle's
    quantization of the same rows (tie-certified: certified groups bit-exact,
    the rest admissible), and the uncertified share is printed;
  * the device reconstruct of the device payload is checked on sampled rows
    against the oracle's exact W_hat of that payload (<= 1e-3 rel-F, <= 1 bf16
    ulp);
  * the device forward of the device payload is checked on sampled rows of x
    against the oracle's exact y (<= 2e-3 rel-F, cos >= 0.9999) and against
    the oracle on the same fp16 operands (<= 1e-5); bf16 y is the RNE of fp32.

The rank-32 factors are inputs both sides share.  For the two 3072-wide
shapes they are the oracle's SVD split of W; for the two 16384 x 6144 shapes,
where the exact SVD takes minutes on the host, they are the recipe's planted
rank-8 component (U sqrt(sigma), V sqrt(sigma) rounded to bf16) padded with
zero columns to rank 32.  The format is exact for any factors.
"""
import time

import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, gen_activations, gen_weight_parts
from tests.helpers import bf16_bits_of, bf16_tensor_to_f64, dev, ulp_bf16

pytestmark = pytest.mark.gpu

Y_TOL, COS_TOL, DIAG_TOL, WHAT_TOL = 2e-3, 0.9999, 1e-5, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4_gemm_amd  # noqa: F401


def _factors(cfg_id, w, u, sig, v):
    cfg = CONFIGS[cfg_id]
    if cfg.N * cfg.K <= 9216 * 3072:
        return O.svd_init(w, cfg.rank)
    up = np.zeros((cfg.N, cfg.rank)); dn = np.zeros((cfg.K, cfg.rank))
    up[:, :len(sig)] = O.bf16_round(u * np.sqrt(sig))
    dn[:, :len(sig)] = O.bf16_round(v * np.sqrt(sig))
    return up, dn


def _bf(a, d):
    return torch.from_numpy(bf16_bits_of(a).view(np.int16)).view(torch.bfloat16).to(d)


@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5])
def test_chain_full_size(cfg_id):
    import w4_gemm_amd as W
    cfg = CONFIGS[cfg_id]
    d = dev()
    rng = np.random.default_rng(0)
    t0 = time.time()
    w, u, sig, v = gen_weight_parts(rng, cfg.N, cfg.K, cfg.spike)
    xbits = gen_activations(rng, cfg.M, cfg.K, cfg.outlier_frac)
    up, dn = _factors(cfg_id, w, u, sig, v)
    print(f"cfg{cfg_id}: inputs and split {time.time() - t0:.1f} s", flush=True)

    p, fidx, flags = W.quantize_weight(torch.from_numpy(w).to(d), _bf(up, d), _bf(dn, d), cfg.group)
    what = W.reconstruct_bf16(p)
    xd = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).to(d)
    y32 = W.linear_fwd(xd, p, torch.float32)
    y16 = W.linear_fwd(xd, p, torch.bfloat16)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0

    # quantizer: sampled weight rows, tie-certified
    srng = np.random.default_rng(cfg_id)
    rows = np.sort(srng.choice(cfg.N, 128, replace=False))
    ri = torch.from_numpy(rows).to(d)
    r = O.residual(w[rows], up[rows], dn)
    res = O.quantize_residual(r, cfg.group)
    qd = O.unpack(p.codes[ri].cpu().numpy())
    sd = p.scales[ri].cpu().numpy().astype(np.float64)
    rep = O.check_device_quant(r, res, cfg.group, qd, sd, fidx[ri].cpu().numpy())
    print(f"cfg{cfg_id} quantize {rep} uncertified share {rep['uncertified'] / rep['groups']:.4f}")
    assert rep["ok"], rep

    # reconstruct of the device payload, on the same sampled rows
    got = bf16_tensor_to_f64(what[ri])
    exact = O.reconstruct(qd, sd, up[rows], dn, cfg.group)
    ref = O.bf16_round(exact)
    e = O.rel_fro(got, ref)
    print(f"cfg{cfg_id} reconstruct relF vs bf16(oracle) {e:.3e}; relF(W_hat, W) "
          f"{O.rel_fro(exact, w[rows]):.4f}")
    assert e <= WHAT_TOL and np.all(np.abs(got - ref) <= ulp_bf16(ref))

    # forward of the device payload, on sampled rows of x (all N outputs)
    y32h = y32.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y32h))
    assert np.array_equal(bf16_tensor_to_f64(y16), O.bf16_round(y32h))
    xr = np.sort(srng.choice(cfg.M, 16, replace=False))
    q_all = O.unpack(p.codes.cpu().numpy())
    s_all = p.scales.cpu().numpy().astype(np.float64)
    x = O.bf16_decode(xbits[xr])
    yref = O.forward(x, q_all, s_all, up, dn, cfg.group)
    ydiag = O.forward_fp16_operands(x, q_all, s_all, up, dn, cfg.group)
    got = y32h[xr]
    e, cs, ed = O.rel_fro(got, yref), O.cosine(got, yref), O.rel_fro(got, ydiag)
    print(f"cfg{cfg_id} forward relF={e:.3e} cos={cs:.7f} vs-fp16-operands={ed:.3e}; "
          f"layer relF vs x W^T {O.rel_fro(got, x @ w.astype(np.float64).T):.4f} "
          f"({time.time() - t0:.1f} s)", flush=True)
    assert e <= Y_TOL and cs >= COS_TOL and ed <= DIAG_TOL
    if cfg.small_m:
        for m in (1, 16):
            ym = W.linear_fwd(xd[:m], p, torch.float32)
            torch.cuda.synchronize()
            gm = ym.cpu().numpy().astype(np.float64)
            xm = O.bf16_decode(xbits[:m])
            rm = O.forward(xm, q_all, s_all, up, dn, cfg.group)
            dm = O.forward_fp16_operands(xm, q_all, s_all, up, dn, cfg.group)
            print(f"cfg{cfg_id} M={m} relF={O.rel_fro(gm, rm):.3e} "
                  f"vs-fp16-operands={O.rel_fro(gm, dm):.3e}")
            assert O.rel_fro(gm, rm) <= Y_TOL and O.rel_fro(gm, dm) <= DIAG_TOL
