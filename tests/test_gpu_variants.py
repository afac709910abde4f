"""GPU parity (C ABI) of the step's variants against the float64 oracle:
packed factor storage, batch-norm layers (diagonal Fisher) in both methods,
the warm-up damping / per-factor refresh schedule, and the weight rescaling.

Tolerances (max |x - y| / max |y| per tensor): 1e-4 for fp32 factors and
updates, 2e-2 for paths with bf16 inputs, 1e-3 for the damped inverses."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import lockstep, say, with_layers

pytestmark = pytest.mark.gpu

FULL_KEYS = ("A", "G", "A_inv", "G_inv", "mom_w", "mom_b", "w", "b", "F_w", "F_b", "dA", "dG")
DIAG_KEYS = ("dA", "dG", "F_w", "F_b", "mom_w", "mom_b", "w", "b")
TOL32 = {"default": 1e-4, "A_inv": 1e-3, "G_inv": 1e-3}
TOL16 = {"default": 2e-2, "A_inv": 1e-3, "G_inv": 1e-3}


def _tall_cfg():
    L = [synth.linear("tall", 70, 45, 20000, bias=True), synth.linear("mid", 300, 260, 700, bias=False)]
    return with_layers(synth.full_config("fc64"), L, steps=2, act_std=1.0, grad_std=1e-2)


@pytest.mark.parametrize("name", ["fc64", "resnet50_kfac", "mlp24_bf16", "pair16k_bf16", "tall"])
def test_packed_factors_lockstep(gpu_lib, name):
    """A and G stored as packed upper triangles: the fp32 SYRK epilogue (FC 64
    and ResNet-50 layer kinds), the split-row reduce (20,000-row factor), the
    register-staged bf16 SYRK (widths not multiples of 8) and the
    direct-to-LDS bf16 SYRK write only the upper entries; the Cholesky reads
    them; lockstep with the oracle."""
    cfg = _tall_cfg() if name == "tall" else synth.small_config(name)
    tol = TOL16 if cfg.act_dtype == "bf16" else TOL32
    lockstep(cfg, min(cfg.steps, 3), tol, FULL_KEYS, packed=True)


@pytest.mark.parametrize("name", ["resnet50_kfac", "pair16k_bf16"])
def test_packed_equals_full_storage(gpu_lib, name):
    """The same two steps in both layouts: the packed factor equals the upper
    triangle of the whole one and every other tensor is equal, bit for bit."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    cfg = synth.small_config(name)
    if name == "resnet50_kfac":
        cfg = with_layers(cfg, list(cfg.layers) + list(_tall_cfg().layers))
    hp = synth.hparams(cfg)
    stacks = {}
    for layout in ("full", "packed"):
        st = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype, factor_layout=layout)
        for li in range(len(cfg.layers)):
            s0 = synth.initial_state(cfg, li)
            if layout == "packed":
                s0 = dict(s0, A=oracle.pack_upper(s0["A"]), G=oracle.pack_upper(s0["G"]))
            st.set_state(li, s0)
        for t in (1, 2):
            for li in range(len(cfg.layers)):
                st.set_inputs(li, synth.step_inputs(cfg, t, li))
            st.step(st.hparams(hp, refresh=True))
        torch.cuda.synchronize()
        assert st.flags() == 0
        stacks[layout] = st
    for li, L in enumerate(cfg.layers):
        a, b = stacks["full"].get_state(li), stacks["packed"].get_state(li)
        for k in a:
            if k in ("A", "G"):
                assert np.array_equal(oracle.pack_upper(a[k]), b[k]), (L.name, k)
            else:
                assert np.array_equal(a[k], b[k]), (L.name, k)
    say(f"{name}: packed and whole factor storage agree bitwise")


def test_schedule_lockstep(gpu_lib):
    """Eight steps whose damping follows a geometric warm-up and whose
    refreshes follow the per-factor schedule (both for 2 steps, then A every
    3rd and G every 2nd): steps that invert only A, only G, both and neither.
    A layer with d_a = d_out puts an A and a G of equal size into one batched
    run that a one-sided refresh splits; a batch-norm layer takes the
    scaled damping.  Damping and refresh bits come from the library's
    schedule on the GPU side and from the oracle's on the other."""
    base = synth.small_config("resnet50_kfac")
    L = list(base.layers[:4]) + [synth.linear("square", 255, 256, 300, bias=True),
                                 synth.batchnorm("bn", 40, 3, 6, 5), base.layers[-1]]
    cfg = with_layers(base, L, steps=8)
    sched = {"damping_init": float(np.float32(0.05)), "damping_target": float(np.float32(2.5e-4)),
             "warmup_steps": 4, "warmup_shape": "geometric", "bn_damping_scale": 8.0, "dense_steps": 2,
             "refresh_every_a": 3, "refresh_every_g": 2}
    pattern = [oracle.schedule(sched, t)[2:] for t in range(1, 9)]
    assert (True, False) in pattern and (False, True) in pattern and (False, False) in pattern
    lockstep(cfg, 8, TOL32, FULL_KEYS, schedule=sched)


@pytest.mark.parametrize("variant", ["full", "diag"])
def test_rescale_lockstep(gpu_lib, variant):
    """Weight rescaling after the update (norm sqrt(2 d_out), bias untouched)
    in both methods, three steps, with conv, linear and batch-norm layers
    (the last not rescaled)."""
    if variant == "full":
        base = synth.small_config("resnet50_kfac")
        L = list(base.layers) + [synth.batchnorm("bn", 12, 2, 7)]
        cfg = with_layers(base, L, rescale=True)
        lockstep(cfg, 3, TOL32, FULL_KEYS)
    else:
        base = synth.small_config("resnet18_diag")
        L = list(base.layers[:6]) + [synth.linear("odd", 13, 7, 30, bias=True), synth.batchnorm("bn", 12, 2, 7),
                                     base.layers[-1]]
        cfg = with_layers(base, L, rescale=True)
        lockstep(cfg, 3, {"default": 1e-4}, DIAG_KEYS)


def test_batchnorm_diag_lockstep(gpu_lib):
    """The diagonal step on ResNet-18 layer kinds with a batch-norm layer after
    every convolution (batch 4 at 64x64: planes of 32x32 down to 2x2, 16-byte
    loads), plus batch-norm layers with odd planes (scalar loads), without a
    beta and with one sample; four steps, damping of batch-norm layers 8x."""
    base = synth.small_config("resnet18_diag")
    L = synth.with_batchnorm(base.layers) + [synth.batchnorm("odd", 5, 3, 5, 7),
                                             synth.batchnorm("gamma_only", 3, 2, 4, bias=False),
                                             synth.batchnorm("one_sample", 2, 1, 3)]
    cfg = with_layers(base, L, steps=4, bn_damping_scale=8.0)
    lockstep(cfg, cfg.steps, {"default": 1e-4}, DIAG_KEYS)


def test_batchnorm_full_lockstep(gpu_lib):
    """The full step on ResNet-50 layer kinds with a batch-norm layer after
    every convolution: conv / FC layers take the Kronecker-factored path,
    batch-norm layers the diagonal one with their own damping; three steps."""
    base = synth.small_config("resnet50_kfac")
    cfg = with_layers(base, synth.with_batchnorm(base.layers), steps=3, bn_damping_scale=8.0)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)
