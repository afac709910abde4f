"""GPU parity of kfac_step_full (C ABI) against the float64 oracle.

Tolerances (max |x - y| / max |y| per tensor): 1e-4 for fp32 factors and
updates, 2e-2 for paths with bf16 inputs, 1e-3 for the damped inverses."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import lockstep, max_rel, say, with_layers

pytestmark = pytest.mark.gpu

FULL_KEYS = ("A", "G", "A_inv", "G_inv", "mom_w", "mom_b", "w", "b")
TOL32 = {"default": 1e-4, "A_inv": 1e-3, "G_inv": 1e-3}
TOL16 = {"default": 2e-2, "A_inv": 1e-3, "G_inv": 1e-3}


def test_fc64_ten_steps(gpu_lib):
    """One FC 64(+bias)->32, batch 128, fp32, inverse every step, 10 steps."""
    cfg = synth.full_config("fc64")
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_resnet50_shapes_small(gpu_lib):
    """ResNet-50 layer kinds at small spatial size: 7x7/2 stem, 3x3, strided
    3x3, 1x1/2 projection, FC with bias; factor sizes 96..1152 (1-9 Cholesky
    blocks, ragged), fewer rows than columns in the FC."""
    cfg = synth.small_config("resnet50_kfac")
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_mlp_bf16_small(gpu_lib):
    """Transformer MLP pair in bf16 (widths not multiples of 8: scalar loads),
    inverse every 2nd step."""
    cfg = synth.small_config("mlp24_bf16")
    lockstep(cfg, cfg.steps, TOL16, FULL_KEYS)


def test_pair_bf16_small(gpu_lib):
    """Large-pair shape family in bf16 (widths multiples of 8: vector loads)."""
    cfg = synth.small_config("pair16k_bf16")
    lockstep(cfg, cfg.steps, TOL16, FULL_KEYS)


def test_fp32_linear_split_k(gpu_lib):
    """Tall-skinny fp32 factors (many rows, few columns) take the split-K path."""
    L = [synth.linear("tall", 70, 45, 20000, bias=True), synth.linear("mid", 300, 260, 700, bias=False)]
    cfg = with_layers(synth.full_config("fc64"), L, steps=2, act_std=1.0, grad_std=1e-2)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_sgd_reduction_update_phase(gpu_lib):
    """UPDATE phase alone with identity inverses: the step is SGD with momentum
    and weight decay (closed form from the oracle's update)."""
    import torch
    from second_order_optimizer_amd import PHASE_UPDATE
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.full_config("fc64"), [synth.linear("fc", 150, 70, 8, bias=True)])
    L = cfg.layers[0]
    st = KfacStack(cfg.layers, "full")
    s0 = synth.initial_state(cfg, 0)
    s0["A_inv"] = np.eye(L.d_a, dtype=np.float32)
    s0["G_inv"] = np.eye(L.d_out, dtype=np.float32)
    st.set_state(0, s0)
    hp = synth.hparams(cfg)
    w = np.concatenate([s0["w"], s0["b"][:, None]], 1).astype(np.float64)
    v = np.zeros_like(w)
    for t in range(1, 4):
        inp = synth.step_inputs(cfg, t, 0)
        st.set_inputs(0, inp)
        st.step(st.hparams(hp, refresh=False, phase_mask=PHASE_UPDATE))
        torch.cuda.synchronize()
        gr = np.concatenate([inp["grad_w"], inp["grad_b"][:, None]], 1).astype(np.float64)
        w, v = oracle.momentum_update(w, v, gr, hp["lr"], hp["momentum"], hp["weight_decay"])
        got = st.get_state(0)
        assert max_rel(got["w"], w[:, :-1]) <= 1e-6 and max_rel(got["b"], w[:, -1]) <= 1e-6
        assert max_rel(got["mom_w"], v[:, :-1]) <= 1e-5 and max_rel(got["mom_b"], v[:, -1]) <= 1e-5


def test_not_pd_keeps_inverse(gpu_lib):
    """A factor with a negative eigenvalue (EMA decay 1 keeps it) fails the
    Cholesky: KFAC_FLAG_NOT_PD is raised and that inverse is left unchanged,
    while the positive definite G is still inverted."""
    import torch
    from second_order_optimizer_amd import FLAG_NOT_PD, PHASE_FACTORS, PHASE_INVERT
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.full_config("fc64"), [synth.linear("fc", 200, 140, 16, bias=True)])
    L = cfg.layers[0]
    st = KfacStack(cfg.layers, "full")
    s0 = synth.initial_state(cfg, 0)
    A = np.eye(L.d_a, dtype=np.float32)
    A[150, 150] = -10 * cfg.damping
    s0["A"] = A
    s0["A_inv"] = np.full((L.d_a, L.d_a), 7.0, np.float32)
    st.set_state(0, s0)
    st.set_inputs(0, synth.step_inputs(cfg, 1, 0))
    hp = dict(synth.hparams(cfg), ema_decay=1.0)
    st.step(st.hparams(hp, refresh=True, phase_mask=PHASE_FACTORS | PHASE_INVERT))
    torch.cuda.synchronize()
    assert st.flags(clear=True) == FLAG_NOT_PD
    got = st.get_state(0)
    assert np.array_equal(got["A_inv"], s0["A_inv"])
    ref = oracle.damped_inverse(np.eye(L.d_out), cfg.damping)
    assert max_rel(got["G_inv"], ref) <= 1e-6


def test_full_deterministic(gpu_lib):
    """Two runs from the same state give bitwise-equal state."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    cfg = synth.small_config("resnet50_kfac")
    res = []
    for _ in range(2):
        st = KfacStack(cfg.layers, "full")
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, 1, li))
        st.step(st.hparams(synth.hparams(cfg), refresh=True))
        torch.cuda.synchronize()
        res.append([st.get_state(li) for li in range(len(cfg.layers))])
    for a, b in zip(*res):
        for k in a:
            assert np.array_equal(a[k], b[k]), k
