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


def lockstep(cfg, steps, tol, check_keys, stack=None, phase_mask=0):
    """Runs `steps` steps of cfg on the GPU (C ABI) and in the oracle, comparing
    every layer's state after each step.  Returns the worst error per key."""
    from second_order_optimizer_amd.stack import KfacStack
    variant = cfg.variant
    if stack is None:
        stack = KfacStack(cfg.layers, variant, cfg.act_dtype, cfg.grad_dtype)
    ostate = []
    for li in range(len(cfg.layers)):
        st = synth.initial_state(cfg, li)
        stack.set_state(li, st)
        ostate.append({k: v.astype(np.float64) for k, v in st.items()})
    hp = synth.hparams(cfg)
    worst = {}
    import torch
    for t in range(1, steps + 1):
        refresh = synth.refresh_at(cfg, t) if variant == "full" else True
        inputs = [synth.step_inputs(cfg, t, li) for li in range(len(cfg.layers))]
        for li in range(len(cfg.layers)):
            stack.set_inputs(li, inputs[li])
        stack.step(stack.hparams(hp, refresh=refresh, phase_mask=phase_mask))
        torch.cuda.synchronize()
        assert stack.flags() == 0, f"device flags raised at step {t}"
        for li, L in enumerate(cfg.layers):
            if variant == "full":
                ref, flags = oracle.step_full(L, ostate[li], inputs[li], hp, refresh)
            else:
                ref, flags = oracle.step_diag(L, ostate[li], inputs[li], hp)
            assert flags == 0
            got = stack.get_state(li)
            for k in check_keys:
                if k not in ref or k not in got:
                    continue
                e = max_rel(got[k], ref[k])
                worst[k] = max(worst.get(k, 0.0), e)
                assert e <= tol.get(k, tol["default"]), f"step {t} layer {li} ({L.name}) {k}: max_rel {e:.3e}"
            ostate[li] = {k: v for k, v in ref.items() if k in ostate[li] or k in ("A_inv", "G_inv")}
        say(f"  step {t}: ok " + " ".join(f"{k}={v:.2e}" for k, v in sorted(worst.items())))
    return worst
