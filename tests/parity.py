"""Helpers shared by the GPU parity tests: the error measure and lockstep
runs of the HIP path (through the C ABI) and the float64 oracle from the same
synthetic state and inputs.  The oracle is never fed anything the HIP path
computed."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle
import synth


def max_rel(x, y) -> float:
    """max |x - y| / max |y| over a tensor (y = oracle); 0 when both are 0."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.abs(y).max() if y.size else 0.0
    num = np.abs(x - y).max() if y.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def with_layers(cfg, layers, **kw):
    return dataclasses.replace(cfg, layers=tuple(layers), **kw)


def oracle_state(cfg, li):
    return {k: v.astype(np.float64) for k, v in synth.initial_state(cfg, li).items()}


def _sched_struct(sched):
    import second_order_optimizer_amd as K
    return K.Schedule(sched["damping_init"], sched["damping_target"], sched["warmup_steps"],
                      K.WARMUP_LINEAR if sched["warmup_shape"] == "linear" else K.WARMUP_GEOMETRIC,
                      sched["bn_damping_scale"], sched["dense_steps"], sched["refresh_every_a"],
                      sched["refresh_every_g"])


def lockstep(cfg, steps, tol, check_keys, stack=None, phase_mask=0, packed=False, schedule=None):
    """Runs `steps` steps of cfg on the GPU (C ABI) and in the oracle, comparing
    every layer's state after each step.  Returns the worst error per key.

    packed: the library keeps A and G as packed upper triangles (set from and
    read back into whole matrices with the oracle's packing).  schedule: a
    dict of oracle.schedule; each step's damping and refresh bits come from
    the library's kfac_schedule_hparams on the GPU side and from
    oracle.schedule on the oracle side (the refresh bits must agree)."""
    import second_order_optimizer_amd as K
    from second_order_optimizer_amd.stack import KfacStack
    variant = cfg.variant
    if stack is None:
        stack = KfacStack(cfg.layers, variant, cfg.act_dtype, cfg.grad_dtype,
                          factor_layout="packed" if packed else "full")
    ostate = []
    for li, L in enumerate(cfg.layers):
        st = synth.initial_state(cfg, li)
        ostate.append({k: v.astype(np.float64) for k, v in st.items()})
        if packed and "A" in st:
            st = dict(st, A=oracle.pack_upper(st["A"]), G=oracle.pack_upper(st["G"]))
        stack.set_state(li, st)
    hp = synth.hparams(cfg)
    worst = {}
    import torch
    for t in range(1, steps + 1):
        hp_t = hp
        if schedule is not None:
            lam, lam_bn, ra, rg = oracle.schedule(schedule, t)
            hp_t = dict(hp, damping=lam, damping_bn=lam_bn)
            refresh = (bool(ra), bool(rg))
            H = K.schedule_hparams(_sched_struct(schedule), t, stack.hparams(hp, phase_mask=phase_mask))
            assert H.refresh == (K.REFRESH_A if ra else 0) | (K.REFRESH_G if rg else 0), (t, H.refresh, ra, rg)
            assert abs(H.damping - lam) <= 1e-6 * lam and abs(H.damping_bn - lam_bn) <= 1e-6 * lam_bn
        else:
            refresh = synth.refresh_at(cfg, t) if variant == "full" else True
            H = stack.hparams(hp, refresh=refresh, phase_mask=phase_mask)
        inputs = [synth.step_inputs(cfg, t, li) for li in range(len(cfg.layers))]
        for li in range(len(cfg.layers)):
            stack.set_inputs(li, inputs[li])
        stack.step(H)
        torch.cuda.synchronize()
        assert stack.flags() == 0, f"device flags raised at step {t}"
        for li, L in enumerate(cfg.layers):
            if variant == "full":
                ref, flags = oracle.step_full(L, ostate[li], inputs[li], hp_t, refresh)
            else:
                ref, flags = oracle.step_diag(L, ostate[li], inputs[li], hp_t)
            assert flags == 0
            got = stack.get_state(li)
            if packed and "A" in got:
                got["A"] = oracle.unpack_upper(got["A"], L.d_a)
                got["G"] = oracle.unpack_upper(got["G"], L.d_out)
            for k in check_keys:
                if k not in ref or k not in got:
                    continue
                e = max_rel(got[k], ref[k])
                worst[k] = max(worst.get(k, 0.0), e)
                assert e <= tol.get(k, tol["default"]), f"step {t} layer {li} ({L.name}) {k}: max_rel {e:.3e}"
            ostate[li] = {k: v for k, v in ref.items() if k in ostate[li] or k in ("A_inv", "G_inv")}
        say(f"  step {t}: ok " + " ".join(f"{k}={v:.2e}" for k, v in sorted(worst.items())))
    return worst
