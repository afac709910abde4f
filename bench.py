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
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
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
    cfg = synth.full_config(args.config)
    log(f"[bench] {cfg.name}: {len(cfg.layers)} layers, {cfg.n_params} params")
    if cfg.variant == "diag":
        res = run_diag(cfg, args)
    else:
        print(f"{cfg.name}: the full K-FAC step is not benchmarked yet", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_diag(cfg)
    line = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic", "config": workload_desc(cfg),
            "roofline": res["roofline"], "cpu_baseline": cpu, "phases": res.get("phases")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
