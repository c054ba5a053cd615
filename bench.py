#!/usr/bin/env python3
"""Throughput of the W4 linear layer's hot path on one MI355X.

One step = the three entry points on one synthetic layer with the inputs
already resident in HBM:
  sq_quantize_weight (rotate + MSE fraction sweep + int4 pack of W),
  sq_linear_fwd      (rotation pre-phase + fused int4 contraction),
  sq_reconstruct_bf16 (bf16 W_hat from the payload).
Each entry point is timed on its own with HIP events on the stream it runs
on (torch's current stream), after warm-up calls.  Every timed loop cycles
through distinct input/output sets of at least 512 MB in total (two whole
forward sets of payload, x, y and workspace; enough payload copies for the
small-M graphs; three reconstruct sets; two quantizer inputs), so the 256 MB
Infinity Cache cannot serve the next call from the previous one, and runs the
same launches back to back for 0.2 s first (after an idle gap the clock ramps
up over the first milliseconds of load).  The headline `value` is the fused
forward's TFLOP/s at 4480x16384x6144 (flops = 2MNK + 2Mr(N+K)); reconstruct
GB/s and quantize GB/s are reported beside it.

The `roofline` object is for the forward's dominant kernel (the contraction,
k_fwd_gemm_big, timed alone through sq_linear_fwd_contract).  Its `traffic`
is the HBM bytes per launch that rocprofv3 counters measured for that kernel
(FETCH_SIZE + WRITE_SIZE, each scaled by the ratio of known bytes to counted
bytes of a plain device copy), read from the committed counter summary under
profiles/; it is null when the kernel source has changed since then.
`cpu_baseline` is the CPU oracle's forward on a sample of rows, on this
host's cores, with the BLAS library and the thread and CPU counts.

Extra fields: the input gradient (sq_linear_dgrad, dx = dy W_hat, same
flop count as the forward, not part of the step), the streaming builder's
wall time on a two-layer fp32 checkpoint, the small-M forward sweep (M = 1, 16, 128 on the
6144x16384 g32 weight) in GB/s of bytes the call must move, the
rotation, reconstruct and quantize kernels against HBM peak, and the
int8-residual mode (rank 16, one int8 code per weight and one fp16 scale
per row) and the MXFP4 mode (rank 32, E2M1 codes with E8M0 block-32
exponents, FP4 x FP4 forward on the scaled MFMA, against the 10.1 PFLOP/s
dense FP4 peak) at the same shape: forward, reconstruct and quantizer.

Context fields: torch's bf16 GEMM (hipBLASLt) on the same activations and the
dense bf16 weight (a comparator only, the on-box counterpart of the pages'
production bf16 GEMM), the oracle's quantizer sweep and reconstruct on a few
sampled weight rows beside its forward, and the current shader and memory
clock levels.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--config 4]
       python bench.py --ops copy      (the counter calibration copy only)
       python bench.py --ops fwd --host-split   (for counter passes: the setup's
                                                 factor split runs on the host)
One JSON line goes to stdout; one progress line per finished section to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6      # MI355X dense fp16/bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense FP4 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PEAK_VALU_TOPS = 39.32        # non-packed vector lane-ops: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
SWEEP_OPS_PER_ELEMENT = 31 * 5
# counter summary of the contraction kernel at 4480x16384x6144 (see its header)
GEMM_PMC = os.path.join(ROOT, "profiles", "k_fwd_gemm_big_mlp-up_4480x16384x6144_pmc.txt")
GEMM_SRC = os.path.join(ROOT, "w4_gemm_amd", "csrc", "sq_fwd.hip")
COPY_BYTES = 256 << 20        # calibration copy: 256 MiB read + 256 MiB written


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(path, src):
    """HBM bytes per launch from a counter summary, or None if it is missing
    or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256_16") != source_sha(src):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def sets_for(set_bytes, rotate_mb):
    """How many distinct sets of `set_bytes` make at least `rotate_mb` MB (at least 2)."""
    return max(2, int(np.ceil(rotate_mb * 1e6 / max(set_bytes, 1.0))))


# set by --host-split: the setup's factor splits run on the host
HOST_SPLIT = False


def split(torch, w, rank, seed=0):
    """bf16 rank-`rank` factors (up [N, r], down [K, r]) of a device weight through
    the builder's seeded fp64 randomized split (on the host under HOST_SPLIT)."""
    from w4_gemm_amd import builder as B
    from w4_gemm_amd.svd_init import _bf16_from_f64
    a = w.double().cpu() if HOST_SPLIT else w.double()
    g = torch.Generator(device=a.device).manual_seed(seed)
    u, s, v = B.randomized_split(torch, a, rank, g)
    rs = s[:rank].sqrt()
    up = _bf16_from_f64((u[:, :rank] * rs).cpu().numpy()).to(w.device)
    down = _bf16_from_f64((v[:, :rank] * rs).cpu().numpy()).to(w.device)
    return up, down


def clone_payload(W, p):
    """A distinct copy of a W4 payload (codes, scales and both factors)."""
    return W.W4Payload(p.codes.clone(), p.scales.clone(),
                       None if p.up is None else p.up.clone(),
                       None if p.down is None else p.down.clone(), p.group)


SETTLE_S = 0.2


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn(i) back to back for `seconds` of wall time before a timed loop.

    After the GPU idles (setup, host work between measurements) its clock
    ramps back up over the first few milliseconds of load, and the very first
    heavy burst of a process has shown one stall of tens of milliseconds;
    the timed steps measure the steady state that follows."""
    t0 = time.perf_counter()
    i = 0
    while True:
        fn(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return


def event_times(torch, fn, steps, warmup):
    """Per-call milliseconds of fn(i) for i = 0..steps-1, HIP events on the
    current stream, after the clock settles and `warmup` untimed calls."""
    settle(torch, fn)
    for i in range(warmup):
        fn(i)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for i, (a, b) in enumerate(marks):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in marks])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4480)
    ap.add_argument("--ops",
                    default="fwd,reconstruct,quantize,dgrad,builder,smallm,configs,w8,mx,bf16gemm")
    ap.add_argument("--small-m", default="1,16,128")
    ap.add_argument("--host-split", action="store_true",
                    help="run the setup's factor splits on the host (for counter passes, where "
                         "the device QR of the split crashes the profiled process)")
    ap.add_argument("--rotate-mb", type=float, default=512.0,
                    help="least total size of the distinct sets a timed loop cycles through")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; the layer shards by output rows "
              "(see the design notes), but no multi-GPU measurement exists.", file=sys.stderr)
        return 2

    import torch

    import w4_gemm_amd as W
    from synth import CONFIGS, f32_to_bf16_bits, gen_activations, gen_weight

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.ops == "copy":
        return copy_calibration(torch, dev)
    cfg = CONFIGS[args.config]
    M, N, K, G, R = cfg.M, cfg.N, cfg.K, cfg.group, cfg.rank
    ops = args.ops.split(",")
    global HOST_SPLIT
    HOST_SPLIT = args.host_split

    # ---------------------------------------------------------------- inputs (untimed)
    t_setup = time.time()
    rng = np.random.default_rng(0)
    w_np = gen_weight(rng, N, K, cfg.spike)
    x_np = gen_activations(rng, M, K, cfg.outlier_frac)
    w = torch.from_numpy(w_np).to(dev)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    del w_np
    # host prerequisite: rank-R factors, from the builder's seeded fp64
    # randomized split (within 1e-4 of the exact SVD's residual energy)
    up, down = split(torch, w, R)
    p0, fidx, flags = W.quantize_weight(w, up, down, G)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0, "quantizer flagged the synthetic weight"
    payloads = [p0] + [clone_payload(W, p0) for _ in range(2)]
    pay_bytes = N * K / 2 + N * (K // G) * 2 + (N + K) * R * 2
    # forward sets: payload, x, y (bf16) and workspace each
    fset_bytes = pay_bytes + M * K * 2 + M * N * 2 + W.fwd_workspace_bytes(M, p0)
    nf = sets_for(fset_bytes, args.rotate_mb)
    xs = [x] + [x.clone() for _ in range(nf - 1)]
    fpays = payloads[:nf] + [clone_payload(W, p0) for _ in range(nf - len(payloads[:nf]))]
    wss = [torch.empty(W.fwd_workspace_bytes(M, p0), dtype=torch.uint8, device=dev) for _ in range(nf)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(nf)]
    what = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def done(section):
        # one progress line per finished section, on stderr (the JSON line is stdout's only line)
        print(f"[bench] {section} done at {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    res = {}
    torch.cuda.synchronize()
    t0 = time.time()
    # ---------------------------------------------------------------- forward
    if "fwd" in ops:
        settle(torch, lambda i: (W.linear_fwd_rotate(xs[i % nf], fpays[i % nf], wss[i % nf]),
                                 W.linear_fwd_contract(M, fpays[i % nf], ys[i % nf], wss[i % nf])))
        for i in range(args.warmup):
            W.linear_fwd_rotate(xs[i % nf], fpays[i % nf], wss[i % nf])
            W.linear_fwd_contract(M, fpays[i % nf], ys[i % nf], wss[i % nf])
        marks = [(ev(), ev(), ev()) for _ in range(args.steps)]
        for i, (a, b, c) in enumerate(marks):
            j = i % nf
            a.record()
            W.linear_fwd_rotate(xs[j], fpays[j], wss[j])
            b.record()
            W.linear_fwd_contract(M, fpays[j], ys[j], wss[j])
            c.record()
        torch.cuda.synchronize()
        rot = np.array([a.elapsed_time(b) for a, b, _ in marks])
        con = np.array([b.elapsed_time(c) for _, b, c in marks])
        res["fwd"] = (rot + con, rot, con)
        res["fwd_sets"] = (nf, fset_bytes * nf)
        # the shader clock while a burst of forwards runs (the idle level differs)
        for i in range(12):
            W.linear_fwd_rotate(xs[i % nf], fpays[i % nf], wss[i % nf])
            W.linear_fwd_contract(M, fpays[i % nf], ys[i % nf], wss[i % nf])
        time.sleep(0.004)
        res["clock_under_load"] = read_clocks()
        torch.cuda.synchronize()
        done("fwd")
    # ---------------------------------------------------------------- reconstruct
    if "reconstruct" in ops:
        res["reconstruct"] = event_times(
            torch, lambda i: W.reconstruct_bf16(payloads[i % 3], out=what[i % 3]), args.steps,
            args.warmup)
        done("reconstruct")
    # ---------------------------------------------------------------- input gradient
    if "dgrad" in ops:
        gen = torch.Generator(device=dev).manual_seed(0)
        dy = torch.randn((M, N), generator=gen, device=dev).to(torch.bfloat16)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dws = torch.empty(W.dgrad_workspace_bytes(M, p0), dtype=torch.uint8, device=dev)
        dps = [p0, payloads[1]]
        res["dgrad"] = event_times(
            torch, lambda i: W.linear_dgrad(dy, dps[i % 2], out=dx, workspace=dws), args.steps,
            args.warmup)
        del dy, dx, dws
        done("dgrad")
    # ---------------------------------------------------------------- quantize
    if "quantize" in ops:
        res["quantize"] = quantize_times(torch, W, dev, [w, w.clone()], up, down, G, args.steps,
                                         args.warmup)
        done("quantize")
    # ---------------------------------------------------------------- int8-residual mode
    if "w8" in ops:
        res["w8"] = w8_run(torch, W, dev, w, x, what, M, N, K, args.steps, args.warmup)
        done("w8")
    # ---------------------------------------------------------------- MXFP4 mode
    if "mx" in ops:
        res["mx"] = mx_run(torch, W, dev, w, x, up, down, what, M, N, K, args.steps, args.warmup)
        done("mx")
    # ---------------------------------------------------------------- comparator
    if "bf16gemm" in ops:
        res["bf16gemm"] = bf16_gemm_run(torch, dev, w, x, M, N, K, args.steps, args.warmup)
        done("bf16gemm")
    # ---------------------------------------------------------------- streaming builder
    if "builder" in ops:
        res["builder"] = builder_run(torch, dev)
        done("builder")
    # ---------------------------------------------------------------- other shapes
    if "configs" in ops:
        res["configs"] = other_configs(torch, W, dev, [1, 2, 3, 5], max(5, args.steps // 5),
                                       args.warmup, args.rotate_mb)
        done("configs")
    # ---------------------------------------------------------------- small-M sweep
    if "smallm" in ops and args.small_m:
        res["smallm"] = small_m_sweep(torch, W, dev, [int(v) for v in args.small_m.split(",")],
                                      args.steps, args.warmup, args.rotate_mb)
        done("smallm")
    torch.cuda.synchronize()
    wall = time.time() - t0

    # ---------------------------------------------------------------- metrics
    flops_fwd = 2.0 * M * N * K + 2.0 * M * R * (N + K)
    flops_gemm = 2.0 * M * N * K + 2.0 * M * N * R
    rec_bytes = pay_bytes + 2.0 * N * K
    quant_bytes = 4.0 * N * K + N * K / 2 + N * (K // G) * 3 + (N + K) * R * 2
    out = {}
    ms_step = 0.0
    if "fwd" in res:
        tot, rot, con = res["fwd"]
        t_fwd, t_rot, t_con = float(np.mean(tot)), float(np.mean(rot)), float(np.mean(con))
        ms_step += t_fwd
        out.update(fwd_ms=t_fwd, fwd_ms_median=float(np.median(tot)),
                   fwd_ms_p10=float(np.percentile(tot, 10)),
                   fwd_ms_p90=float(np.percentile(tot, 90)), fwd_rotate_ms=t_rot,
                   fwd_contract_ms=t_con, fwd_tflops=flops_fwd / (t_fwd * 1e-3) / 1e12)
        out["fwd_pct_bf16_mfma_peak"] = 100.0 * out["fwd_tflops"] / PEAK_F16_TFLOPS
        out["fwd_rotating_sets"] = {"sets": res["fwd_sets"][0], "bytes": res["fwd_sets"][1]}
        # rotation half: reads x twice, writes xh (fp16); the t / stats side buffers are small
        rot_bytes = 3.0 * M * K * 2
        out["fwd_rotate_gbps"] = rot_bytes / (t_rot * 1e-3) / 1e9
        achieved = flops_gemm / (t_con * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": "k_fwd_gemm_big", "achieved": achieved,
                           "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / PEAK_F16_TFLOPS,
                           "traffic": measured_traffic(GEMM_PMC, GEMM_SRC),
                           "per_launch_flops": flops_gemm,
                           "algorithmic_bytes_per_launch": M * K * 2 + pay_bytes + M * N * 2}
    if "reconstruct" in res:
        t = float(np.mean(res["reconstruct"]))
        ms_step += t
        out.update(reconstruct_ms=t, reconstruct_ms_median=float(np.median(res["reconstruct"])),
                   reconstruct_gbps=rec_bytes / (t * 1e-3) / 1e9)
        out["reconstruct_pct_hbm_peak"] = 100.0 * out["reconstruct_gbps"] / PEAK_HBM_GBPS
    if "quantize" in res:
        t = float(np.mean(res["quantize"]["times"]))
        ms_step += t
        out.update(quantize_ms=t, quantize_gbps=quant_bytes / (t * 1e-3) / 1e9)
        out["quantize_pct_hbm_peak"] = 100.0 * out["quantize_gbps"] / PEAK_HBM_GBPS
        # the 31-candidate sweep is plain fp32 ALU work: 5 lane-ops per element
        # and candidate (multiply, round, clamp, two FMAs), against the
        # non-packed vector issue rate of 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
        alu = SWEEP_OPS_PER_ELEMENT * N * K / (t * 1e-3)
        out["quantize_alu"] = {"bound": "alu", "achieved": alu / 1e12, "peak": PEAK_VALU_TOPS,
                               "unit": "Tlane-op/s", "frac": alu / 1e12 / PEAK_VALU_TOPS,
                               "ops_per_element": SWEEP_OPS_PER_ELEMENT}
        out["quantize_other_configs"] = res["quantize"]["other"]
    if "dgrad" in res:
        t = float(np.mean(res["dgrad"]))
        out.update(dgrad_ms=t, dgrad_ms_median=float(np.median(res["dgrad"])),
                   dgrad_tflops=flops_fwd / (t * 1e-3) / 1e12)
        out["dgrad_pct_bf16_mfma_peak"] = 100.0 * out["dgrad_tflops"] / PEAK_F16_TFLOPS
    if "builder" in res:
        out["builder"] = res["builder"]
    if "w8" in res:
        out["w8"] = res["w8"]
    if "mx" in res:
        out["mx"] = res["mx"]
    if "bf16gemm" in res:
        out["bf16_gemm_hipblaslt"] = res["bf16gemm"]
    if "smallm" in res:
        out["fwd_small_m"] = res["smallm"]
    if "configs" in res:
        out["fwd_other_configs"] = res["configs"]

    line = {
        "metric": "fused W4 fwd TFLOP/s (% bf16 MFMA peak) at 4480x16384x6144; reconstruct GB/s",
        "value": out.get("fwd_tflops"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} rank{R}", "M": M, "N": N, "K": K, "group": G,
                   "rank": R, "out_dtype": "bf16"},
        "roofline": out.pop("roofline", None),
        "cpu_baseline": None,
    }
    line.update({k: v for k, v in out.items()})
    line["timed_wall_s"] = wall
    line["settle_s_per_timed_loop"] = SETTLE_S
    line["setup_s"] = t_setup
    line["device"] = torch.cuda.get_device_name(0)
    line["clocks"] = read_clocks()
    if "clock_under_load" in res:
        line["clocks_under_load"] = res["clock_under_load"]

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p0, x, cfg, args.cpu_rows)
        line["cpu_baseline_other"] = cpu_other(p0, w, cfg)
    print(json.dumps(line), flush=True)
    return 0


def w8_run(torch, W, dev, w, x, what, M, N, K, steps, warmup):
    """The int8-residual mode at the same layer shape with rank-16 factors:
    sq_quantize_weight_w8 of the same weight, then sq_linear_fwd_w8 (whole
    call: rotation pre-phase + int8 contraction) and sq_reconstruct_bf16_w8
    (rotating over three payload/output sets), each timed with HIP events."""
    R = 16
    up, down = split(torch, w, R)
    qws = torch.empty(W._lib.sq_quantize_weight_w8_workspace_bytes(W.empty_payload_w8(N, K, R, dev).abi()),
                      dtype=torch.uint8, device=dev)
    p0, fidx, flags = W.quantize_weight_w8(w, up, down, workspace=qws)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0, "int8 quantizer flagged the synthetic weight"
    pays = [p0] + [W.W8Payload(p0.codes.clone(), p0.scales.clone(), up, down) for _ in range(2)]
    ws = torch.empty(W.fwd_w8_workspace_bytes(M, p0), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def done(section):
        # one progress line per finished section, on stderr (the JSON line is stdout's only line)
        print(f"[bench] {section} done at {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    def timed(fn):
        return float(np.mean(event_times(torch, fn, steps, warmup)))

    y2, x2 = torch.empty_like(y), x.clone()
    t_fwd = timed(lambda i: W.linear_fwd_w8(x if i % 2 else x2, pays[i % 3], out=y if i % 2 else y2,
                                            workspace=ws))
    t_rec = timed(lambda i: W.reconstruct_bf16_w8(pays[i % 3], out=what[i % 3]))
    t_q = timed(lambda i: W.quantize_weight_w8(w, up, down, want_fidx=False, workspace=qws))
    flops = 2.0 * M * N * K + 2.0 * M * R * (N + K)
    pay = N * K + 2.0 * N + (N + K) * R * 2
    rec_bytes = pay + 2.0 * N * K
    out = {"rank": R, "fwd_ms": t_fwd, "fwd_tflops": flops / (t_fwd * 1e-3) / 1e12,
           "reconstruct_ms": t_rec, "reconstruct_gbps": rec_bytes / (t_rec * 1e-3) / 1e9,
           "quantize_ms": t_q}
    out["fwd_pct_bf16_mfma_peak"] = 100.0 * out["fwd_tflops"] / PEAK_F16_TFLOPS
    out["reconstruct_pct_hbm_peak"] = 100.0 * out["reconstruct_gbps"] / PEAK_HBM_GBPS
    npay = sets_for(pay, 512.0)
    spays = pays[:npay] + [W.W8Payload(p0.codes.clone(), p0.scales.clone(), up, down)
                           for _ in range(npay - len(pays[:npay]))]
    out["fwd_small_m"] = small_m_modes(
        torch, dev, x, N, K, pay, steps, warmup,
        lambda m: W.fwd_w8_workspace_bytes(m, p0),
        lambda i, xx, yy, wss: W.linear_fwd_w8(xx, spays[i % npay], out=yy, workspace=wss))
    out["fwd_small_m"]["payload_copies"] = npay
    del pays, spays, p0, qws, ws, y, y2, x2
    torch.cuda.empty_cache()
    return out


def mx_run(torch, W, dev, w, x, up, down, what, M, N, K, steps, warmup):
    """The MXFP4 mode at the same layer shape with the same rank-32 factors:
    sq_quantize_weight_mx4 of the same weight, then sq_linear_fwd_mx4 (whole
    call: activation rotation + FP4 quantization + low-rank projection, FP4
    contraction) and sq_reconstruct_bf16_mx4 (rotating over three
    payload/output sets), each timed with HIP events."""
    R = up.shape[1]
    p0, flags = W.quantize_weight_mx4(w, up, down)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0, "FP4 quantizer flagged the synthetic weight"
    pays = [p0] + [W.MX4Payload(p0.codes.clone(), p0.exps.clone(), up, down) for _ in range(2)]
    ws = torch.empty(W.fwd_mx4_workspace_bytes(M, p0), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def done(section):
        # one progress line per finished section, on stderr (the JSON line is stdout's only line)
        print(f"[bench] {section} done at {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    def timed(fn):
        return float(np.mean(event_times(torch, fn, steps, warmup)))

    y2, x2 = torch.empty_like(y), x.clone()
    t_fwd = timed(lambda i: W.linear_fwd_mx4(x if i % 2 else x2, pays[i % 3], out=y if i % 2 else y2,
                                             workspace=ws))
    t_rec = timed(lambda i: W.reconstruct_bf16_mx4(pays[i % 3], out=what[i % 3]))
    t_q = timed(lambda i: W.quantize_weight_mx4(w, up, down))
    flops = 2.0 * M * N * K + 2.0 * M * R * (N + K)
    pay = N * K / 2 + N * K / 32 + (N + K) * R * 2
    rec_bytes = pay + 2.0 * N * K
    out = {"rank": R, "fwd_ms": t_fwd, "fwd_tflops": flops / (t_fwd * 1e-3) / 1e12,
           "reconstruct_ms": t_rec, "reconstruct_gbps": rec_bytes / (t_rec * 1e-3) / 1e9,
           "quantize_ms": t_q}
    out["fwd_pct_fp4_mfma_peak"] = 100.0 * out["fwd_tflops"] / PEAK_FP4_TFLOPS
    out["reconstruct_pct_hbm_peak"] = 100.0 * out["reconstruct_gbps"] / PEAK_HBM_GBPS
    npay = sets_for(pay, 512.0)
    spays = pays[:npay] + [W.MX4Payload(p0.codes.clone(), p0.exps.clone(), up, down)
                           for _ in range(npay - len(pays[:npay]))]
    out["fwd_small_m"] = small_m_modes(
        torch, dev, x, N, K, pay, steps, warmup,
        lambda m: W.fwd_mx4_workspace_bytes(m, p0),
        lambda i, xx, yy, wss: W.linear_fwd_mx4(xx, spays[i % npay], out=yy, workspace=wss))
    out["fwd_small_m"]["payload_copies"] = npay
    del pays, spays, p0, ws, y, y2, x2
    torch.cuda.empty_cache()
    return out


def graph_us(torch, fn, steps, warmup):
    """GPU time per call of fn(i), in microseconds, from one replay of a HIP
    graph of `steps` back-to-back calls i = 0..steps-1 (small calls finish
    faster than the host enqueues them, so eager timing would measure the
    host)."""
    settle(torch, fn)
    for i in range(warmup):
        fn(i)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                fn(i)
    torch.cuda.synchronize()
    settle(torch, lambda i: graph.replay())
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps * 1e3


def small_m_modes(torch, dev, x, N, K, pay, steps, warmup, ws_bytes, fwd, ms=(1, 16, 128)):
    """Forward of the int8 or MXFP4 payload at small M (first M rows of the
    layer's activations), graph-replayed with consecutive calls on distinct
    payload copies; GB/s of payload + x + y."""
    out = {}
    for m in ms:
        xm = x[:m].contiguous()
        y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(ws_bytes(m), dtype=torch.uint8, device=dev)
        t = graph_us(torch, lambda i: fwd(i, xm, y, ws), steps, warmup)
        by = pay + m * K * 2 + m * N * 2
        out[str(m)] = {"us": t, "gbps": by / (t * 1e-6) / 1e9,
                       "pct_hbm_peak": 100.0 * by / (t * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    return out


def copy_calibration(torch, dev, reps=5):
    """Plain device copies of known size, for scaling the HBM byte counters:
    torch's copy_ (the runtime's blit kernel) and an elementwise kernel
    (b = a * 1, vector loads and stores like the library's kernels), each
    reading COPY_BYTES and writing COPY_BYTES."""
    n = COPY_BYTES // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / reps
    t = time.perf_counter()
    for _ in range(reps):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    dt2 = (time.perf_counter() - t) / reps
    print(json.dumps({"calibration_copy_bytes_read": COPY_BYTES, "calibration_copy_bytes_written":
                      COPY_BYTES, "blit_ms": dt * 1e3, "elementwise_ms": dt2 * 1e3}), flush=True)
    return 0


def builder_run(torch, dev):
    """The streaming builder end to end on a synthetic two-layer checkpoint
    (the MLP-up and MLP-down weights, fp32, 16384x6144 and 6144x16384 g32
    rank 32, randomized SVD) in a temporary directory: wall seconds and
    source GB/s, SVD, quantizer and file writes included."""
    import shutil
    import tempfile

    from safetensors.torch import save_file

    from w4_gemm_amd import builder as B
    from synth import gen_weight
    tmp = tempfile.mkdtemp(prefix="sq_builder_")
    try:
        rng = np.random.default_rng(0)
        src = os.path.join(tmp, "model.safetensors")
        save_file({"mlp.up.weight": torch.from_numpy(gen_weight(rng, 16384, 6144, 8)),
                   "mlp.down.weight": torch.from_numpy(gen_weight(rng, 6144, 16384, 8))}, src)
        src_bytes = os.path.getsize(src)
        torch.cuda.synchronize()
        t = time.perf_counter()
        out = B.build(src, os.path.join(tmp, "slab"), rank=32, group=32, svd="randomized")
        dt = time.perf_counter() - t
        return {"seconds": dt, "source_bytes": src_bytes, "slab_bytes": os.path.getsize(out),
                "source_gbps": src_bytes / dt / 1e9,
                "workload": "2 fp32 weights 16384x6144 + 6144x16384, g32 rank 32"}
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def layer(torch, W, dev, cfg_id, with_w=False):
    """Synthetic layer of a configuration: its payload (quantized on the GPU
    with the seeded rank-R split) and its activation draw (numpy bf16)."""
    from synth import CONFIGS, gen_activations, gen_weight
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng(0)
    w = torch.from_numpy(gen_weight(rng, cfg.N, cfg.K, cfg.spike)).to(dev)
    x_all = gen_activations(rng, cfg.M, cfg.K, cfg.outlier_frac)
    up, down = split(torch, w, cfg.rank)
    p, _, flags = W.quantize_weight(w, up, down, cfg.group)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0
    return (cfg, p, x_all, w) if with_w else (cfg, p, x_all)


def quantize_times(torch, W, dev, ws_in, up, down, G, steps, warmup):
    """sq_quantize_weight on the headline weight (cycling through the given
    copies of it) and, as extra rows, on the fused-QKV weight (9216 x 3072
    g64) and the tiny layer, each cycling through >= 512 MB of inputs."""
    from w4_gemm_amd import _lib
    stream = torch.cuda.current_stream().cuda_stream

    def runner(wl, upl, dnl, group):
        n, k = wl[0].shape
        qp = W.empty_payload(n, k, group, upl.shape[1], dev)
        qp.up, qp.down = upl, dnl
        abi = qp.abi()
        qf = torch.empty((n, k // group), dtype=torch.uint8, device=dev)
        flags = torch.zeros(4, dtype=torch.int32, device=dev)

        def go(i):
            st = _lib.sq_quantize_weight(wl[i % len(wl)].data_ptr(), abi, qf.data_ptr(),
                                         flags.data_ptr(), stream)
            assert st == 0, st
        return go

    times = event_times(torch, runner(ws_in, up, down, G), steps, warmup)
    other = {}
    from synth import CONFIGS, gen_weight
    for cid in (3, 1):
        cfg = CONFIGS[cid]
        w = torch.from_numpy(gen_weight(np.random.default_rng(0), cfg.N, cfg.K, cfg.spike)).to(dev)
        u, d = split(torch, w, cfg.rank)
        nb = 4.0 * cfg.N * cfg.K + cfg.N * cfg.K / 2 + cfg.N * (cfg.K // cfg.group) * 3 + \
            (cfg.N + cfg.K) * cfg.rank * 2
        wl = [w] + [w.clone() for _ in range(sets_for(nb, 512.0) - 1)]
        t = float(np.mean(event_times(torch, runner(wl, u, d, cfg.group), steps, warmup)))
        other[cfg.name] = {"us": t * 1e3, "gbps": nb / (t * 1e-3) / 1e9,
                           "pct_hbm_peak": 100.0 * nb / (t * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                           "rotating_sets": len(wl)}
        del wl, w
    torch.cuda.empty_cache()
    return {"times": times, "other": other}


def other_configs(torch, W, dev, ids, steps, warmup, rotate_mb):
    """The whole forward at the other layer shapes (their own M), and the
    reconstruct at the shapes whose text names it (attention projection,
    MLP-down, tiny), timed per call with HIP events on the current stream,
    each loop cycling through >= rotate_mb MB of distinct sets."""
    out = {}
    for cid in ids:
        cfg, p, x_all = layer(torch, W, dev, cid)
        M, N, K, G, R = cfg.M, cfg.N, cfg.K, cfg.group, cfg.rank
        pay = N * K / 2 + N * (K // G) * 2 + (N + K) * R * 2
        fb = pay + M * K * 2 + M * N * 2 + W.fwd_workspace_bytes(M, p)
        nf = sets_for(fb, rotate_mb)
        pays = [p] + [clone_payload(W, p) for _ in range(nf - 1)]
        x0 = torch.from_numpy(x_all.view(np.int16)).view(torch.bfloat16).to(dev)
        xs = [x0] + [x0.clone() for _ in range(nf - 1)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(nf)]
        wss = [torch.empty(W.fwd_workspace_bytes(M, p), dtype=torch.uint8, device=dev)
               for _ in range(nf)]
        t = float(np.median(event_times(
            torch, lambda i: W.linear_fwd(xs[i % nf], pays[i % nf], out=ys[i % nf],
                                          workspace=wss[i % nf]), steps, warmup)))
        fl = 2.0 * M * N * K + 2.0 * M * R * (N + K)
        row = {"us": t * 1e3, "tflops": fl / (t * 1e-3) / 1e12,
               "pct_mfma_peak": 100.0 * fl / (t * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
               "rotating_sets": nf}
        del xs, ys, wss
        if cid in (1, 2, 5):
            rb = pay + 2.0 * N * K
            nr = sets_for(rb, rotate_mb)
            rp = pays[:nr] + [clone_payload(W, p) for _ in range(nr - len(pays[:nr]))]
            outs = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(nr)]
            tr = float(np.mean(event_times(
                torch, lambda i: W.reconstruct_bf16(rp[i % nr], out=outs[i % nr]), steps, warmup)))
            row["reconstruct"] = {"us": tr * 1e3, "gbps": rb / (tr * 1e-3) / 1e9,
                                  "pct_hbm_peak": 100.0 * rb / (tr * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                  "rotating_sets": nr}
            del rp, outs
        out[cfg.name] = row
        del p, pays
        torch.cuda.empty_cache()
    return out


def small_m_sweep(torch, W, dev, ms, steps, warmup, rotate_mb=512.0):
    """Forward at small M on the 6144x16384 g32 rank-32 weight, HBM-bound:
    GB/s of the bytes one call must move (payload + x + y), first M rows of
    the M=4480 activation draw.  At these sizes one call's kernels run for
    less time than the host needs to enqueue them, so the calls are captured
    once in a HIP graph and the graph is replayed: the figure is GPU time
    per call (`us`), with the eager per-call time beside it (`eager_us`).
    Consecutive calls use distinct payload copies (>= rotate_mb MB in all),
    so no call finds its payload in the Infinity Cache."""
    cfg, p, x_all = layer(torch, W, dev, 5)
    N, K, G, R = cfg.N, cfg.K, cfg.group, cfg.rank
    pay = N * K / 2 + N * (K // G) * 2 + (N + K) * R * 2
    npay = sets_for(pay, rotate_mb)
    pays = [p] + [clone_payload(W, p) for _ in range(npay - 1)]
    out = {"payload_copies": npay}
    for m in ms:
        x = torch.from_numpy(x_all[:m].view(np.int16).copy()).view(torch.bfloat16).to(dev)
        y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(W.fwd_workspace_bytes(m, p), dtype=torch.uint8, device=dev)
        eager = float(np.median(event_times(
            torch, lambda i: W.linear_fwd(x, pays[i % npay], out=y, workspace=ws), steps, warmup)))
        # graph: `steps` calls captured back to back on a side stream
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                for i in range(steps):
                    W.linear_fwd(x, pays[i % npay], out=y, workspace=ws)
        torch.cuda.synchronize()
        settle(torch, lambda i: graph.replay())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / steps
        by = pay + m * K * 2 + m * N * 2
        out[str(m)] = {"us": t * 1e3, "eager_us": eager * 1e3, "gbps": by / (t * 1e-3) / 1e9,
                       "pct_hbm_peak": 100.0 * by / (t * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                       "tflops": (2.0 * m * N * K + 2.0 * m * R * (N + K)) / (t * 1e-3) / 1e12}
    del pays
    torch.cuda.empty_cache()
    return out


def bf16_gemm_run(torch, dev, w, x, M, N, K, steps, warmup):
    """Comparator only (not a code path): torch's bf16 GEMM (hipBLASLt) of the
    same activations with the dense bf16 weight, y = x @ W^T, at the same
    shape; the on-box counterpart of the pages' production bf16 GEMM column."""
    wt = w.t().contiguous().to(torch.bfloat16)   # [K, N], no transposed view
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = float(np.mean(event_times(torch, lambda i: torch.mm(x, wt, out=y), steps, warmup)))
    del wt, y
    torch.cuda.empty_cache()
    return {"ms": t, "tflops": 2.0 * M * N * K / (t * 1e-3) / 1e12}


def read_clocks():
    """Current shader and memory clock levels as the driver lists them (best effort)."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device"))[:1]:
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [l.strip() for l in f if l.strip().endswith("*")]
                out[name] = cur[0] if cur else None
            except OSError:
                out[name] = None
    return out


def cpu_other(p, w, cfg, rows=1024):
    """The oracle's quantizer (the 31-fraction sweep of the rotated residual,
    without the SVD) and reconstruct on `rows` sampled weight rows."""
    import oracle as O
    sel = np.sort(np.random.default_rng(2).choice(cfg.N, rows, replace=False))
    wr = w[sel].cpu().numpy().astype(np.float64)
    up = p.up.float().cpu().numpy().astype(np.float64)
    dn = p.down.float().cpu().numpy().astype(np.float64)
    r = O.residual(wr, up[sel], dn)
    t = time.perf_counter()
    res = O.quantize_residual(r, cfg.group)
    t_q = time.perf_counter() - t
    codes = p.codes[torch_index(sel, p.codes)].cpu().numpy()
    scales = p.scales[torch_index(sel, p.scales)].cpu().numpy()
    t = time.perf_counter()
    wh = O.reconstruct(O.unpack(codes), O.fp16_decode(scales), up[sel], dn, cfg.group)
    t_r = time.perf_counter() - t
    assert np.all(np.isfinite(wh)) and res.q.shape == (rows, cfg.K)
    elems = rows * cfg.K
    return {"quantize_sweep": {"value": elems / t_q / 1e6, "unit": "Melem/s", "seconds": t_q,
                               "sample": f"oracle.quantize_residual on {rows} of {cfg.N} rows, K={cfg.K}"},
            "reconstruct": {"value": elems / t_r / 1e6, "unit": "Melem/s", "seconds": t_r,
                            "sample": f"oracle.reconstruct on {rows} of {cfg.N} rows, K={cfg.K}"}}


def torch_index(sel, t):
    import torch
    return torch.from_numpy(sel).to(t.device)


def cpu_baseline(p, x, cfg, rows):
    """The oracle's forward on `rows` sampled rows of x against the full payload."""
    import oracle as O
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        if info:
            blas = {"vendor": info[0].get("internal_api"), "version": info[0].get("version"),
                    "threading": info[0].get("threading_layer"),
                    "architecture": info[0].get("architecture")}
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    codes = p.codes.cpu().numpy()
    scales = p.scales.cpu().numpy()
    up = p.up.float().cpu().numpy().astype(np.float64)
    dn = p.down.float().cpu().numpy().astype(np.float64)
    sel = np.sort(np.random.default_rng(1).choice(cfg.M, rows, replace=False))
    xs = x[sel].float().cpu().numpy().astype(np.float64)
    t = time.perf_counter()
    q = O.unpack(codes)
    y = O.forward(xs, q, O.fp16_decode(scales), up, dn, cfg.group)
    dt = time.perf_counter() - t
    assert np.all(np.isfinite(y))
    flops = 2.0 * rows * cfg.N * cfg.K + 2.0 * rows * cfg.rank * (cfg.N + cfg.K)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle.forward (numpy fp64) on {rows} of {cfg.M} rows, full N={cfg.N} "
                      f"K={cfg.K}, including unpack/dequant; {dt:.2f} s",
            "seconds": dt, "blas": blas, "os_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    sys.exit(main())
