#!/usr/bin/env python3
"""Optimizer-step throughput of the HIP K-FAC library on one MI355X.

A step is one call of the library's step entry point over the whole layer
stack of a synthetic workload, inputs already resident in HBM.  The default
run measures all five workloads in one process and prints ONE JSON line:
`value` is the diagonal (AdaFisher-style) step over the ResNet-18 parameter
set, batch 128 at 224x224; `configs` holds every workload's steps/s, per-phase
times, TFLOP/s against the MFMA peak of its dtype (full K-FAC) or GB/s
against HBM (diagonal), and the float64 CPU oracle timed on the host.
`--config NAME` measures one workload alone.

Phases are timed live with HIP events on the stream the library launches on
(single-phase calls through the C ABI).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_TFLOPS = 157.3       # dense fp32 MFMA
BF16_MFMA_TFLOPS = 2500.0      # dense bf16 MFMA

METRIC = "K-FAC steps/s per layer stack; factor+precond TFLOP/s (%MFMA); diag-step GB/s"
HEADLINE = "resnet18_diag"
ORDER = ("resnet18_diag", "fc64", "resnet50_kfac", "mlp24_bf16", "pair16k_bf16", "resnet50_bn_diag")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "diag_resnet18_b128_traffic.md")
DIAG_SRC = os.path.join(ROOT, "second_order_optimizer_amd", "csrc", "diag.hip")
COPY_BYTES = 1 << 30     # the --traffic-probe calibration copy reads and writes 1 GiB


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_desc(cfg) -> dict:
    d = {"workload": cfg.name, "variant": cfg.variant, "layers": len(cfg.layers), "params": cfg.n_params,
         "act_dtype": cfg.act_dtype, "grad_dtype": cfg.grad_dtype}
    d["desc"] = {
        "resnet18_diag": "ResNet-18 shapes (20 conv + FC 512->1000), batch 128 @ 224x224, diagonal step",
        "resnet50_kfac": "ResNet-50 shapes (53 conv + FC 2048->1000), batch 32 @ 224x224, full K-FAC, invert every step",
        "mlp24_bf16": "24 x (1024->4096, 4096->1024) linears with bias, 8192 tokens, bf16 a/g, invert every 10",
        "pair16k_bf16": "4096->16384 and 16384->4096 linears with bias, 16384 tokens, bf16 a/g, invert every 20",
        "fc64": "one FC 64(+1)->32, batch 128, full K-FAC, invert every step",
        "resnet50_bn_diag": "the 53 batch-norm layers of ResNet-50 at batch 32 @ 224x224 (gamma, beta per channel), "
                            "diagonal Fisher step",
    }[cfg.name]
    d["refresh_every"] = cfg.refresh_every if cfg.variant == "full" else None
    return d


# ---------------------------------------------------------------------------
# algorithmic work

def diag_factor_bytes(cfg) -> int:
    """Algorithmic bytes of the diagonal FACTORS phase (a7): every element of a
    and g read once (4 B), dA and dG written once."""
    import numpy as np
    n = 0
    for L in cfg.layers:
        n += 4 * (int(np.prod(L.act_shape)) + int(np.prod(L.grad_out_shape)))
        n += 4 * (2 * L.d_out if L.kind == "bn" else L.d_a + L.d_out)
    return n


def rescale_bytes(cfg) -> int:
    """Algorithmic bytes of the weight rescaling: every conv / linear weight
    read twice (norm, then scale) and written once, 12 B per weight."""
    return 12 * sum(L.d_out * L.d_in for L in cfg.layers if L.kind != "bn")


def diag_update_bytes(cfg) -> int:
    """Algorithmic bytes of the diagonal parameter pass (a8): grad, W, V, F read
    and W, V, F written, 4 B each (28 B per parameter)."""
    return 28 * cfg.n_params


def full_flops(layers):
    """Algorithmic flops of the full step per layer stack: SYRK (upper
    triangle with diagonal, 2 flops per multiply-add: rows * d * (d + 1)),
    preconditioning (2 d_g^2 d_a + 2 d_g d_a^2) and the damped inverse
    (POTRF + TRTRI + LAUUM, d^3 / 3 each)."""
    syrk = sum(L.rows * d * (d + 1) for L in layers for d in (L.d_a, L.d_out))
    pre = sum(2 * L.d_out ** 2 * L.d_a + 2 * L.d_out * L.d_a ** 2 for L in layers)
    inv = sum(L.d_a ** 3 + L.d_out ** 3 for L in layers)
    return syrk, pre, inv


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host

def host_info():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def _timed(fn):
    """Runs fn() with the BLAS pool at all host cores; (wall s, cpu s, cores)."""
    from threadpoolctl import threadpool_limits
    cores, _ = host_info()
    with threadpool_limits(limits=cores, user_api="blas"):
        c0, t0 = time.process_time(), time.perf_counter()
        fn()
        wall, cpu = time.perf_counter() - t0, time.process_time() - c0
    return wall, cpu, cores


def cpu_baseline_diag(cfg):
    """The oracle's whole diagonal step over every layer at the workload's full
    size (one step)."""
    import oracle
    import synth
    hp = synth.hparams(cfg)
    data = [(synth.initial_state(cfg, li), synth.step_inputs(cfg, 1, li)) for li in range(len(cfg.layers))]

    def run():
        for li, L in enumerate(cfg.layers):
            oracle.step_diag(L, data[li][0], data[li][1], hp)
    wall, cpu, cores = _timed(run)
    _, model = host_info()
    return {"value": 1.0 / wall, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle, one whole diagonal step over all {len(cfg.layers)} layers at full size "
                      f"(batch {cfg.layers[0].batch}): {wall:.2f} s wall, {cpu:.1f} s CPU; BLAS pool of {cores} "
                      f"threads on {model}"}


def cpu_sample(cfg):
    """(layer indices, row divisor) of the full method's CPU sample; the FC 64
    workload runs whole."""
    n = len(cfg.layers)
    if cfg.name == "mlp24_bf16":
        return [0, 1], 1                   # one of 24 identical blocks
    if cfg.name == "pair16k_bf16":
        return [0], 8                      # the 4096->16384 layer at 2048 of 16384 tokens
    if cfg.name == "resnet50_kfac":
        return [0, 7, 20, 33, 46, n - 1], 1   # stem, 3x3 convs of each stage, FC
    return list(range(n)), 1


def cpu_baseline_full(cfg):
    """The oracle's full step: the FC 64 workload's ten steps whole; the larger
    stacks on a sample of their layers, once as a refresh step and once as a
    stale step, the amortised time scaled to the whole stack by the ratio of
    algorithmic flops (labelled as a sample)."""
    import dataclasses
    import numpy as np
    import oracle
    import synth
    hp = synth.hparams(cfg)
    _, model = host_info()
    if cfg.name == "fc64":
        L = cfg.layers[0]
        st0 = {k: v.astype(np.float64) for k, v in synth.initial_state(cfg, 0).items()}
        inputs = [synth.step_inputs(cfg, t, 0) for t in range(1, cfg.steps + 1)]

        def run():
            st = st0
            for t, inp in enumerate(inputs, 1):
                out, _ = oracle.step_full(L, st, inp, hp, synth.refresh_at(cfg, t))
                st = {k: out[k] for k in st0}
        wall, cpu, cores = _timed(run)
        return {"value": cfg.steps / wall, "unit": "steps/s", "cores": cores, "kind": "oracle",
                "sample": f"float64 numpy oracle, all {cfg.steps} steps of the workload: {wall * 1e3:.1f} ms wall; "
                          f"BLAS pool of {cores} threads on {model}"}
    idx, div = cpu_sample(cfg)
    sub = [cfg.layers[i] if div == 1 else dataclasses.replace(cfg.layers[i], rows=cfg.layers[i].rows // div)
           for i in idx]
    scfg = dataclasses.replace(cfg, layers=tuple(sub))
    data = [(synth.initial_state(scfg, j), synth.step_inputs(scfg, 1, j)) for j in range(len(sub))]
    times = {}
    cpu_total = 0.0
    for refresh in (True, False):
        def run():
            for (st, inp), L in zip(data, sub):
                oracle.step_full(L, st, inp, hp, refresh)
        times[refresh], cpu, cores = _timed(run)
        cpu_total += cpu
    k = cfg.refresh_every
    t_sample = (times[True] + (k - 1) * times[False]) / k
    fs, fp, fi = full_flops(sub)
    ts, tp, ti = full_flops(cfg.layers)
    scale = (ts + tp + ti / k) / (fs + fp + fi / k)
    return {"value": 1.0 / (t_sample * scale), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"SAMPLE: float64 numpy oracle, full step on layers {idx} of {len(cfg.layers)}"
                      f"{'' if div == 1 else f' at 1/{div} of the rows'}: refresh step {times[True]:.2f} s, stale "
                      f"step {times[False]:.2f} s wall ({cpu_total:.1f} s CPU), amortised over a refresh interval "
                      f"of {k}, scaled x{scale:.2f} to the whole stack by algorithmic flops; BLAS pool of {cores} "
                      f"threads on {model}"}


# ---------------------------------------------------------------------------
# GPU runs

def _load(cfg, pool):
    import synth
    from second_order_optimizer_amd.stack import KfacStack
    st = KfacStack(cfg.layers, cfg.variant, cfg.act_dtype, cfg.grad_dtype, pool=pool)
    for li in range(len(cfg.layers)):
        st.set_state(li, synth.initial_state(cfg, li))
    for slot in range(pool):
        for li in range(len(cfg.layers)):
            st.set_inputs(li, synth.step_inputs(cfg, slot + 1, li), slot=slot)
        log(f"[bench] {cfg.name}: input batch {slot + 1}/{pool} resident")
    return st


def _time_phase(st, hp, pool, mask, n, refresh=False):
    """Average time (ms) of `n` back-to-back calls that run only `mask`,
    between two HIP events recorded on the stream the library launches on
    (torch's current stream); one event pair around the whole run keeps the
    events' own cost out of short phases."""
    import torch
    Hm = st.hparams(hp, refresh=refresh, phase_mask=mask)
    stream = torch.cuda.current_stream()
    st.step(Hm)                      # one untimed call: the phase's first launches are warm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        st.use_inputs(i % pool)
        st.step(Hm)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def run_diag(cfg, args):
    import torch
    import synth
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_RESCALE, PHASE_UPDATE
    pool = max(1, args.pool)
    st = _load(cfg, pool)
    hp = synth.hparams(cfg)
    H = st.hparams(hp)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        st.use_inputs(i % pool)
        st.step(H)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.use_inputs(i % pool)
        st.step(H)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    log(f"[bench] {cfg.name}: timed {args.steps} steps: {ms:.3f} ms/step")
    nk = max(5, args.steps)
    t_fac = _time_phase(st, hp, pool, PHASE_FACTORS, nk)
    t_upd = _time_phase(st, hp, pool, PHASE_UPDATE, nk)
    rb = rescale_bytes(cfg)
    t_resc = _time_phase(st, dict(hp, rescale=True), pool, PHASE_RESCALE, nk) if rb else None
    assert st.flags() == 0, "device flags raised"
    del st
    torch.cuda.empty_cache()
    fb, ub = diag_factor_bytes(cfg), diag_update_bytes(cfg)
    gbs = lambda b, t: b / (t * 1e-3) / 1e9
    bn = all(L.kind == "bn" for L in cfg.layers)
    out = {
        "ms_per_step": ms, "steps_per_s": 1e3 / ms, "steps": args.steps, "dtype": "f32",
        "a7_diag_factors": {"kernels": "diag_bn_kernel" if bn else "diag_colsq_kernel + diag_finish_kernel",
                            "ms": t_fac, "bytes": fb, "GBps": gbs(fb, t_fac), "peak_GBps": HBM_PEAK_GBS,
                            "frac": gbs(fb, t_fac) / HBM_PEAK_GBS},
        "a8_diag_step": {"kernels": "diag_update_kernel", "ms": t_upd, "bytes": ub, "GBps": gbs(ub, t_upd),
                         "peak_GBps": HBM_PEAK_GBS, "frac": gbs(ub, t_upd) / HBM_PEAK_GBS},
        "step_GBps": gbs(fb + ub, ms),
    }
    if rb:
        out["rescale"] = {"kernels": "rescale_norm_kernel + rescale_apply_kernel", "ms": t_resc, "bytes": rb,
                          "GBps": gbs(rb, t_resc), "frac": gbs(rb, t_resc) / HBM_PEAK_GBS}
    return out


def run_full(cfg, args):
    import torch
    import synth
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_INVERT, PHASE_RESCALE, PHASE_UPDATE, REFRESH_A, REFRESH_G
    from second_order_optimizer_amd.stack import KfacStack
    pool = max(1, args.pool)
    st = _load(cfg, pool)
    hp = synth.hparams(cfg)
    k = cfg.refresh_every
    steps = max(k, (args.steps + k - 1) // k * k)     # whole refresh intervals
    H = {r: st.hparams(hp, refresh=r) for r in (True, False)}
    torch.cuda.synchronize()
    for i in range(max(1, args.warmup)):
        st.use_inputs(i % pool)
        st.step(H[i % k == 0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st.use_inputs(i % pool)
        st.step(H[i % k == 0])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / steps
    log(f"[bench] {cfg.name}: timed {steps} steps: {ms:.3f} ms/step")
    n = max(3, min(10, args.steps))
    t_fac = _time_phase(st, hp, pool, PHASE_FACTORS, n)
    t_inv = _time_phase(st, hp, pool, PHASE_INVERT, max(2, n // 3), refresh=True)
    t_inv_a = _time_phase(st, hp, pool, PHASE_INVERT, max(2, n // 3), refresh=REFRESH_A)
    t_inv_g = _time_phase(st, hp, pool, PHASE_INVERT, max(2, n // 3), refresh=REFRESH_G)
    t_upd = _time_phase(st, hp, pool, PHASE_UPDATE, n)
    rb = rescale_bytes(cfg)
    t_resc = _time_phase(st, dict(hp, rescale=True), pool, PHASE_RESCALE, n)
    assert st.flags() == 0, "device flags raised"
    # the factor phase again with A and G stored as packed upper triangles
    # (same input buffers; factor contents do not affect the timing)
    pk = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype, factor_layout="packed", inputs_from=st)
    t_fac_packed = _time_phase(pk, hp, pool, PHASE_FACTORS, n)
    del pk, st
    torch.cuda.empty_cache()
    fs, fp, fi = full_flops(cfg.layers)
    syrk_peak = BF16_MFMA_TFLOPS if cfg.act_dtype == "bf16" else FP32_MFMA_TFLOPS
    tf = lambda f, t: f / (t * 1e-3) / 1e12
    out = {
        "ms_per_step": ms, "steps_per_s": 1e3 / ms, "steps": steps, "refresh_every": k, "dtype": cfg.act_dtype,
        "factors": {"ms": t_fac, "flops": fs, "tflops": tf(fs, t_fac), "peak_tflops": syrk_peak,
                    "frac": tf(fs, t_fac) / syrk_peak, "dtype": cfg.act_dtype},
        "precond_update": {"ms": t_upd, "flops": fp, "tflops": tf(fp, t_upd), "peak_tflops": FP32_MFMA_TFLOPS,
                           "frac": tf(fp, t_upd) / FP32_MFMA_TFLOPS, "dtype": "f32"},
        "invert": {"ms": t_inv, "amortised_ms": t_inv / k, "flops": fi, "tflops": tf(fi, t_inv),
                   "peak_tflops": FP32_MFMA_TFLOPS, "frac": tf(fi, t_inv) / FP32_MFMA_TFLOPS, "dtype": "f32",
                   "A_only_ms": t_inv_a, "G_only_ms": t_inv_g},
        "factors_packed": {"ms": t_fac_packed, "tflops": tf(fs, t_fac_packed),
                           "frac": tf(fs, t_fac_packed) / syrk_peak,
                           "ema_bytes_whole": 8 * sum(L.d_a ** 2 + L.d_out ** 2 for L in cfg.layers),
                           "ema_bytes_packed": 4 * sum(L.d_a * (L.d_a + 1) + L.d_out * (L.d_out + 1)
                                                       for L in cfg.layers)},
        "rescale": {"kernels": "rescale_norm_kernel + rescale_apply_kernel", "ms": t_resc, "bytes": rb,
                    "GBps": rb / (t_resc * 1e-3) / 1e9, "frac": rb / (t_resc * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    ideal = fs / (syrk_peak * 1e12) + fp / (FP32_MFMA_TFLOPS * 1e12)
    out["combined_mfma_frac"] = ideal / ((t_fac + t_upd) * 1e-3)
    return out


# ---------------------------------------------------------------------------
# counter-measured traffic of the headline workload's FACTORS phase

def _function_text(src, name):
    """Source text of the first __global__ / __device__ definition of `name`."""
    m = re.search(r"(__global__|__device__)[^;{]*?\b" + re.escape(name) + r"\s*\(", src)
    if not m:
        return ""
    i = src.index("{", m.end())
    depth = 0
    for j in range(i, len(src)):
        depth += {"{": 1, "}": -1}.get(src[j], 0)
        if depth == 0:
            return src[m.start():j + 1]
    return src[m.start():]


A7_KERNELS = ("diag_colsq_kernel", "dpp_mov", "wave_sum", "tap_mask", "fin_window", "fin_window_block",
              "diag_finish_kernel")


def a7_source_sha256():
    src = open(DIAG_SRC).read()
    return hashlib.sha256("\n".join(_function_text(src, n) for n in A7_KERNELS).encode()).hexdigest()


def measured_traffic():
    """HBM bytes per FACTORS call of the headline workload (both a7 kernels)
    from the committed counter summary, or None when it is missing or the
    kernels' source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("    ") and ":" in line:
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("a7_kernels_sha256") != a7_source_sha256():
        return None
    try:
        return int(vals["a7_traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def traffic_probe(args):
    """What the FETCH_SIZE / WRITE_SIZE passes profile: a plain 1 GiB device
    copy (calibration of the counters), then `--steps` FACTORS-only diagonal
    calls on ResNet-18 @ 128 (diag_colsq_kernel, diag_finish_kernel) and
    `--steps` UPDATE-only calls (diag_update_kernel)."""
    import torch
    import synth
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_UPDATE
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    cfg = synth.full_config(HEADLINE)
    st = _load(cfg, 1)
    for mask in (PHASE_FACTORS, PHASE_UPDATE):
        H = st.hparams(synth.hparams(cfg), phase_mask=mask)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            st.step(H)
        torch.cuda.synchronize()
    print(json.dumps({"probe": "traffic", "copy_bytes": COPY_BYTES, "factor_calls": args.steps,
                      "update_calls": args.steps, "a7_kernels_sha256": a7_source_sha256()}), flush=True)


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="all", help="all (default) or one of " + ", ".join(ORDER))
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
    names = ORDER if args.config == "all" else (args.config,)
    if any(n not in synth.CONFIG_NAMES for n in names):
        print(f"unknown config {args.config}; choose all or one of {synth.CONFIG_NAMES}", file=sys.stderr)
        sys.exit(2)
    if args.traffic_probe:
        traffic_probe(args)
        return

    results = {}
    for name in names:
        cfg = synth.full_config(name)
        log(f"[bench] {cfg.name}: {len(cfg.layers)} layers, {cfg.n_params} params")
        res = run_diag(cfg, args) if cfg.variant == "diag" else run_full(cfg, args)
        res["config"] = workload_desc(cfg)
        if not args.no_cpu_baseline:
            log(f"[bench] {cfg.name}: timing the CPU oracle")
            res["cpu_baseline"] = cpu_baseline_diag(cfg) if cfg.variant == "diag" else cpu_baseline_full(cfg)
        results[name] = res

    head = HEADLINE if HEADLINE in results else names[0]
    h = results[head]
    if "a7_diag_factors" in h:
        d = h["a7_diag_factors"]
        roof = {"bound": "hbm", "kernel": "a7 diagonal factors: " + d["kernels"], "achieved": d["GBps"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["frac"],
                "traffic": measured_traffic() if head == HEADLINE else None,
                "bytes_per_launch": d["bytes"], "avg_launch_ms": d["ms"]}
    else:
        phases = {p: h[p] for p in ("factors", "precond_update", "invert")}
        dom = max(phases, key=lambda p: phases[p]["ms"] / (h["refresh_every"] if p == "invert" else 1))
        d = phases[dom]
        roof = {"bound": "mfma", "kernel": dom, "achieved": d["tflops"], "peak": d["peak_tflops"], "unit": "TFLOP/s",
                "frac": d["frac"], "traffic": None, "flops_per_launch": d["flops"], "avg_launch_ms": d["ms"]}
    line = {"metric": METRIC, "value": h["steps_per_s"], "unit": "steps/s", "n_gpus": 1, "steps": h["steps"],
            "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": h["dtype"], "data": "synthetic", "config": h["config"],
            "roofline": roof, "cpu_baseline": h.get("cpu_baseline"),
            "configs": {n: {k: v for k, v in r.items() if k != "config"} for n, r in results.items()}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
