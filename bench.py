#!/usr/bin/env python3
"""Optimizer-step throughput of the HIP K-FAC library on one MI355X.

A step is one call of the library's step entry point over the whole layer
stack of a synthetic workload, inputs already resident in HBM.  The default
workload is the diagonal (AdaFisher-style) step over a ResNet-18 parameter
set, batch 128 at 224x224; ``--config`` selects the other workloads.

Prints one JSON line (rank 0) with steps/s, the roofline position of the
dominant kernel (timed live with HIP events on the stream it runs on) and the
float64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_TFLOPS = 157.3       # dense fp32 MFMA
BF16_MFMA_TFLOPS = 2500.0      # dense bf16 MFMA

METRIC = "K-FAC steps/s per layer stack; factor+precond TFLOP/s (%MFMA); diag-step GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "diag_colsq_resnet18_b128_traffic.md")
DIAG_SRC = os.path.join(ROOT, "second_order_optimizer_amd", "csrc", "diag.hip")
COPY_BYTES = 1 << 30     # the --traffic-probe calibration copy reads and writes 1 GiB


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_desc(cfg) -> dict:
    import synth
    d = {"workload": cfg.name, "variant": cfg.variant, "layers": len(cfg.layers), "params": cfg.n_params,
         "act_dtype": cfg.act_dtype, "grad_dtype": cfg.grad_dtype}
    if cfg.name == "resnet18_diag":
        d["desc"] = "ResNet-18 shapes (20 conv + FC 512->1000), batch 128 @ 224x224, diagonal step"
    elif cfg.name == "resnet50_kfac":
        d["desc"] = "ResNet-50 shapes (53 conv + FC 2048->1000), batch 32 @ 224x224, full K-FAC, invert every step"
    elif cfg.name == "mlp24_bf16":
        d["desc"] = "24 x (1024->4096, 4096->1024) linears with bias, 8192 tokens, bf16 a/g, invert every 10"
    elif cfg.name == "pair16k_bf16":
        d["desc"] = "4096->16384 and 16384->4096 linears with bias, 16384 tokens, bf16 a/g, invert every 20"
    elif cfg.name == "fc64":
        d["desc"] = "one FC 64(+1)->32, batch 128, full K-FAC, invert every step"
    d["refresh_every"] = cfg.refresh_every if cfg.variant == "full" else None
    return d


def diag_factor_bytes(cfg) -> int:
    """Algorithmic bytes of the diagonal FACTORS launch: every element of a and
    g read once (4 B), dA and dG written once."""
    import numpy as np
    n = 0
    for L in cfg.layers:
        n += 4 * (int(np.prod(L.act_shape)) + int(np.prod(L.grad_out_shape)))
        n += 4 * (L.d_a + L.d_out)
    return n


def diag_update_bytes(cfg) -> int:
    """Algorithmic bytes of the diagonal parameter pass: grad, W, V, F read and
    W, V, F written, 4 B each (28 B per parameter)."""
    return 28 * cfg.n_params


def cpu_baseline_diag(cfg_full, seconds_target=15.0):
    """The oracle's diagonal step over every layer of the workload at a reduced
    batch; the oracle's cost is linear in the batch, so the full-batch step
    time is the sample time scaled by batch / sample batch."""
    import numpy as np
    import oracle
    import synth
    full_batch = cfg_full.layers[0].batch
    sb = 16
    layers = synth.resnet18_layers(batch=sb)
    cfg = synth.Config(cfg_full.cfg_id, cfg_full.name, "diag", tuple(layers), 1, cfg_full.lr, cfg_full.momentum,
                       cfg_full.weight_decay, cfg_full.ema_decay, cfg_full.damping, act_std=cfg_full.act_std,
                       grad_std=cfg_full.grad_std, relu=cfg_full.relu)
    hp = synth.hparams(cfg)
    data = [(synth.initial_state(cfg, li), synth.step_inputs(cfg, 1, li)) for li in range(len(layers))]
    t0, c0 = time.perf_counter(), time.process_time()
    for li, L in enumerate(layers):
        oracle.step_diag(L, data[li][0], data[li][1], hp)
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    step_s = wall * full_batch / sb
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": max(1, int(round(cpu / max(wall, 1e-9)))),
            "kind": "oracle",
            "sample": f"float64 numpy oracle, diagonal step over all {len(layers)} layers at batch {sb} "
                      f"(full workload batch {full_batch}); measured {wall:.2f} s, scaled x{full_batch // sb} "
                      f"(cost linear in batch)"}


def full_flops(layers):
    """Algorithmic flops of the full step per layer stack: SYRK (upper
    triangle with diagonal, 2 flops per multiply-add: rows * d * (d + 1)),
    preconditioning (2 d_g^2 d_a + 2 d_g d_a^2) and the damped inverse
    (POTRF + TRTRI + LAUUM, d^3 / 3 each)."""
    syrk = sum(L.rows * d * (d + 1) for L in layers for d in (L.d_a, L.d_out))
    pre = sum(2 * L.d_out ** 2 * L.d_a + 2 * L.d_out * L.d_a ** 2 for L in layers)
    inv = sum(L.d_a ** 3 + L.d_out ** 3 for L in layers)
    return syrk, pre, inv


def cpu_sample_layers(cfg):
    """(layer indices, row divisor) of the CPU-baseline sample."""
    n = len(cfg.layers)
    if cfg.name == "mlp24_bf16":
        return [0, 1], 1                   # one of 24 identical blocks
    if cfg.name == "pair16k_bf16":
        return [0], 8                      # the 4096->16384 layer at 2048 of 16384 tokens
    if cfg.name == "resnet50_kfac":
        return [0, 7, 20, 33, 46, n - 1], 1   # stem, 3x3 convs of each stage, FC
    return list(range(n)), 1


def cpu_baseline_full(cfg):
    """The oracle's full step timed on a subset of the stack's layers, once as a
    refresh step and once as a stale step; the amortised sample time is scaled
    to the whole stack by the ratio of algorithmic flops."""
    import dataclasses
    import oracle
    import synth
    idx, div = cpu_sample_layers(cfg)
    sub = [cfg.layers[i] if div == 1 else dataclasses.replace(cfg.layers[i], rows=cfg.layers[i].rows // div)
           for i in idx]
    scfg = dataclasses.replace(cfg, layers=tuple(sub))
    hp = synth.hparams(cfg)
    data = [(synth.initial_state(scfg, j), synth.step_inputs(scfg, 1, j)) for j in range(len(sub))]
    times = {}
    c0 = time.process_time()
    w0 = time.perf_counter()
    for refresh in (True, False):
        t0 = time.perf_counter()
        for (st, inp), L in zip(data, sub):
            oracle.step_full(L, st, inp, hp, refresh)
        times[refresh] = time.perf_counter() - t0
    wall = time.perf_counter() - w0
    cpu = time.process_time() - c0
    k = cfg.refresh_every
    t_sample = (times[True] + (k - 1) * times[False]) / k
    fs, fp, fi = full_flops(sub)
    ts, tp, ti = full_flops(cfg.layers)
    scale = (ts + tp + ti / k) / (fs + fp + fi / k)
    step_s = t_sample * scale
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": max(1, int(round(cpu / max(wall, 1e-9)))),
            "kind": "oracle",
            "sample": f"float64 numpy oracle, full step on layers {idx} of {len(cfg.layers)}"
                      f"{'' if div == 1 else f' at 1/{div} of the rows'}: refresh step "
                      f"{times[True]:.2f} s, stale step {times[False]:.2f} s, amortised over a refresh interval "
                      f"of {k}, scaled x{scale:.2f} by algorithmic flops"}


def run_full(cfg, args):
    import torch
    import synth
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_INVERT, PHASE_UPDATE
    from second_order_optimizer_amd.stack import KfacStack

    pool = max(1, args.pool)
    st = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype, pool=pool)
    for li in range(len(cfg.layers)):
        st.set_state(li, synth.initial_state(cfg, li))
    for slot in range(pool):
        for li in range(len(cfg.layers)):
            st.set_inputs(li, synth.step_inputs(cfg, slot + 1, li), slot=slot)
        log(f"[bench] input batch {slot + 1}/{pool} resident")
    hp = synth.hparams(cfg)
    k = cfg.refresh_every
    steps = max(k, (args.steps + k - 1) // k * k)     # whole refresh intervals
    H = {r: st.hparams(hp, refresh=r) for r in (True, False)}
    torch.cuda.synchronize()
    for i in range(max(1, args.warmup)):
        st.use_inputs(i % pool)
        st.step(H[i % k == 0])
    torch.cuda.synchronize()
    log("[bench] warmup done")
    t0 = time.perf_counter()
    for i in range(steps):
        st.use_inputs(i % pool)
        st.step(H[i % k == 0])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / steps
    log(f"[bench] timed {steps} steps: {ms:.3f} ms/step")
    stream = torch.cuda.current_stream()

    def time_phase(mask, n, refresh=False):
        Hm = st.hparams(hp, refresh=refresh, phase_mask=mask)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            st.use_inputs(i % pool)
            evs[i][0].record(stream)
            st.step(Hm)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n

    n = max(3, min(10, args.steps))
    t_fac = time_phase(PHASE_FACTORS, n)
    t_inv = time_phase(PHASE_INVERT, max(2, n // 3), refresh=True)
    t_upd = time_phase(PHASE_UPDATE, n)
    assert st.flags() == 0, "device flags raised"
    fs, fp, fi = full_flops(cfg.layers)
    syrk_peak = BF16_MFMA_TFLOPS if cfg.act_dtype == "bf16" else FP32_MFMA_TFLOPS
    tf = lambda f, t: f / (t * 1e-3) / 1e12
    phases = {
        "factors": {"ms": t_fac, "tflops": tf(fs, t_fac), "peak": syrk_peak, "frac": tf(fs, t_fac) / syrk_peak,
                    "flops": fs, "dtype": cfg.act_dtype},
        "precond_update": {"ms": t_upd, "tflops": tf(fp, t_upd), "peak": FP32_MFMA_TFLOPS,
                           "frac": tf(fp, t_upd) / FP32_MFMA_TFLOPS, "flops": fp, "dtype": "f32"},
        "invert": {"ms": t_inv, "amortised_ms": t_inv / k, "tflops": tf(fi, t_inv), "peak": FP32_MFMA_TFLOPS,
                   "frac": tf(fi, t_inv) / FP32_MFMA_TFLOPS, "flops": fi, "dtype": "f32"},
    }
    ideal = fs / (syrk_peak * 1e12) + fp / (FP32_MFMA_TFLOPS * 1e12)
    phases["combined_mfma_frac"] = ideal / ((t_fac + t_upd) * 1e-3)
    dom = max(("factors", t_fac), ("precond_update", t_upd), ("invert", t_inv / k), key=lambda x: x[1])[0]
    names = {"factors": "factor SYRK + EMA launches (im2col, syrk_bf16_kernel / gemm_f32_kernel EPI_SYRK, split reduce)",
             "precond_update": "preconditioning GEMMs (gemm_f32_kernel, STORE then fused UPDATE epilogue)",
             "invert": "blocked Cholesky inverse launches"}
    d = phases[dom]
    roof = {"bound": "mfma", "kernel": names[dom], "achieved": d["tflops"], "peak": d["peak"], "unit": "TFLOP/s",
            "frac": d["frac"], "traffic": None, "flops_per_launch": d["flops"], "avg_launch_ms": d["ms"]}
    return {"value": 1e3 / ms, "unit": "steps/s", "ms_per_step": ms, "dtype": cfg.act_dtype,
            "roofline": roof, "phases": phases, "steps": steps}


def source_sha256(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of diag_colsq_kernel from the committed counter
    summary, or None when it is missing or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("    ") and ":" in line:
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_sha256(DIAG_SRC):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_probe(args):
    """What the FETCH_SIZE / WRITE_SIZE passes profile: a plain 1 GiB device
    copy (calibration of the counters), then `--steps` FACTORS-only diagonal
    calls on ResNet-18 @ 128 (each one launch of diag_colsq_kernel) and
    `--steps` UPDATE-only calls (diag_finish_kernel, diag_update_kernel)."""
    import torch
    import synth
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_UPDATE
    from second_order_optimizer_amd.stack import KfacStack
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    cfg = synth.full_config("resnet18_diag")
    st = KfacStack(cfg.layers, "diag")
    for li in range(len(cfg.layers)):
        st.set_state(li, synth.initial_state(cfg, li))
        st.set_inputs(li, synth.step_inputs(cfg, 1, li))
    H = st.hparams(synth.hparams(cfg), phase_mask=PHASE_FACTORS)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        st.step(H)
    torch.cuda.synchronize()
    Hu = st.hparams(synth.hparams(cfg), phase_mask=PHASE_UPDATE)
    for _ in range(args.steps):
        st.step(Hu)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "traffic", "copy_bytes": COPY_BYTES, "factor_calls": args.steps,
                      "update_calls": args.steps, "diag_src_sha256": source_sha256(DIAG_SRC)}), flush=True)


def run_diag(cfg, args):
    import torch
    import synth
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_UPDATE
    from second_order_optimizer_amd.stack import KfacStack

    pool = max(1, args.pool)
    st = KfacStack(cfg.layers, "diag", pool=pool)
    for li in range(len(cfg.layers)):
        st.set_state(li, synth.initial_state(cfg, li))
    for slot in range(pool):
        for li in range(len(cfg.layers)):
            st.set_inputs(li, synth.step_inputs(cfg, slot + 1, li), slot=slot)
        log(f"[bench] input batch {slot + 1}/{pool} resident")
    hp = synth.hparams(cfg)
    H_all = st.hparams(hp)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        st.use_inputs(i % pool)
        st.step(H_all)
    torch.cuda.synchronize()
    log("[bench] warmup done")
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.use_inputs(i % pool)
        st.step(H_all)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps: {dt * 1e3 / args.steps:.3f} ms/step")

    # live per-kernel timing with HIP events on the stream the library uses
    stream = torch.cuda.current_stream()

    def time_phase(mask, n):
        H = st.hparams(hp, phase_mask=mask)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            st.use_inputs(i % pool)
            evs[i][0].record(stream)
            st.step(H)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n   # ms

    nk = max(5, args.steps)
    t_fac = time_phase(PHASE_FACTORS, nk)
    t_upd = time_phase(PHASE_UPDATE, nk)
    assert st.flags() == 0, "device flags raised"
    fb = diag_factor_bytes(cfg)
    ub = diag_update_bytes(cfg)
    ms = dt * 1e3 / args.steps
    achieved = fb / (t_fac * 1e-3) / 1e9
    out = {
        "value": 1e3 / ms, "unit": "steps/s", "ms_per_step": ms, "dtype": "f32",
        "roofline": {"bound": "hbm", "kernel": "diag_colsq_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "bytes_per_launch": fb, "avg_launch_ms": t_fac},
        "phases": {"factors_ms": t_fac, "update_ms": t_upd,
                   "update_GBps": ub / (t_upd * 1e-3) / 1e9,
                   "step_GBps": (fb + ub) / (ms * 1e-3) / 1e9},
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="resnet18_diag")
    ap.add_argument("--pool", type=int, default=2, help="pre-loaded input batches cycled by the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only what the FETCH_SIZE / WRITE_SIZE counter passes measure")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this library "
              "implements the single-GPU optimizer step; multi-GPU sharding is a design note only.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import second_order_optimizer_amd as kfac
    kfac.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.config not in synth.CONFIG_NAMES:
        print(f"unknown config {args.config}; choose from {synth.CONFIG_NAMES}", file=sys.stderr)
        sys.exit(2)
    if args.traffic_probe:
        traffic_probe(args)
        return
    cfg = synth.full_config(args.config)
    log(f"[bench] {cfg.name}: {len(cfg.layers)} layers, {cfg.n_params} params")
    if cfg.variant == "diag":
        res = run_diag(cfg, args)
    else:
        res = run_full(cfg, args)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_diag(cfg) if cfg.variant == "diag" else cpu_baseline_full(cfg)
    line = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
            "steps": res.get("steps", args.steps),
            "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic", "config": workload_desc(cfg),
            "roofline": res["roofline"], "cpu_baseline": cpu, "phases": res.get("phases")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
