"""GPU parity of kfac_step_diag (C ABI) against the float64 oracle.

Tolerance: max |x - y| / max |y| <= 1e-4 per tensor (fp32 arithmetic)."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import lockstep, max_rel, say, with_layers

pytestmark = pytest.mark.gpu

TOL = {"default": 1e-4}
DIAG_KEYS = ("dA", "dG", "F_w", "F_b", "mom_w", "mom_b", "w", "b")


def test_diag_resnet18_small(gpu_lib):
    """ResNet-18 layer kinds at batch 4, 64x64 input: 20 convs (7x7/2 stem,
    3x3, 1x1/2 projections) + FC 512->1000 with bias; 3 steps."""
    cfg = synth.small_config("resnet18_diag")
    say("resnet18 small diag", len(cfg.layers), "layers")
    lockstep(cfg, cfg.steps, TOL, DIAG_KEYS)


def test_diag_edge_shapes(gpu_lib):
    """Odd widths (scalar paths), more rows than one reduction chunk, a 1-row
    layer, conv with bias, a 1x1 stride-2 conv on an odd plane."""
    L = [synth.linear("odd_chunked", 7, 5, 1300, bias=True),
         synth.linear("one_row", 64, 33, 1, bias=True),
         synth.linear("nobias", 12, 8, 9, bias=False),
         synth.conv("stem_odd", 3, 5, 7, 2, 3, 3, 9),
         synth.conv("proj", 4, 6, 1, 2, 0, 2, 7),
         synth.conv("biased", 2, 3, 3, 1, 1, 2, 5, bias=True)]
    cfg = with_layers(synth.small_config("resnet18_diag"), L, steps=4)
    lockstep(cfg, cfg.steps, TOL, DIAG_KEYS)


def test_diag_window_kernel_sizes(gpu_lib):
    """Every kernel size the ABI accepts besides 1, 3 and 7 (2, 4, 5, 6, with
    strides 1-3 and padding beyond the kernel's half-width), a plane large
    enough for eight wavefronts per window item, and a plane wider than
    2048 columns (tap masks computed per pixel instead of from tables)."""
    L = [synth.conv("k2", 3, 4, 2, 2, 0, 2, 9, 11),
         synth.conv("k4", 2, 3, 4, 1, 2, 2, 8),
         synth.conv("k5", 3, 2, 5, 3, 2, 2, 13, 10),
         synth.conv("k6", 2, 5, 6, 2, 3, 2, 9, 7),
         synth.conv("big_plane", 2, 3, 3, 1, 1, 2, 96, 100),
         synth.conv("wide", 1, 2, 3, 2, 1, 2, 3, 2100, bias=True)]
    cfg = with_layers(synth.small_config("resnet18_diag"), L, steps=2)
    lockstep(cfg, cfg.steps, TOL, DIAG_KEYS)


def test_diag_phase_split_equals_fused(gpu_lib):
    """FACTORS then UPDATE as two calls gives the same bits as one call."""
    import torch
    from second_order_optimizer_amd import PHASE_FACTORS, PHASE_UPDATE
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.small_config("resnet18_diag"),
                      [synth.conv("c", 8, 16, 3, 2, 1, 4, 12), synth.linear("fc", 40, 10, 4)])
    outs = []
    for split in (False, True):
        st = KfacStack(cfg.layers, "diag")
        for li in range(2):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, 1, li))
        hp = synth.hparams(cfg)
        if split:
            st.step(st.hparams(hp, phase_mask=PHASE_FACTORS))
            st.step(st.hparams(hp, phase_mask=PHASE_UPDATE))
        else:
            st.step(st.hparams(hp))
        torch.cuda.synchronize()
        outs.append([st.get_state(li) for li in range(2)])
    for a, b in zip(*outs):
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_diag_deterministic(gpu_lib):
    """Two runs from the same state give bitwise-equal results."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    cfg = synth.small_config("resnet18_diag")
    res = []
    for _ in range(2):
        st = KfacStack(cfg.layers, "diag")
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, 1, li))
        st.step(st.hparams(synth.hparams(cfg)))
        torch.cuda.synchronize()
        res.append([st.get_state(li) for li in range(len(cfg.layers))])
    for a, b in zip(*res):
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_diag_nonfinite_flag(gpu_lib):
    """A NaN gradient raises KFAC_FLAG_NONFINITE (forced from the host)."""
    import torch
    from second_order_optimizer_amd import FLAG_NONFINITE
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.small_config("resnet18_diag"), [synth.linear("fc", 16, 8, 4)])
    st = KfacStack(cfg.layers, "diag")
    st.set_state(0, synth.initial_state(cfg, 0))
    inp = synth.step_inputs(cfg, 1, 0)
    inp["grad_w"] = inp["grad_w"].copy()
    inp["grad_w"][3, 5] = np.nan
    st.set_inputs(0, inp)
    st.step(st.hparams(synth.hparams(cfg)))
    torch.cuda.synchronize()
    assert st.flags(clear=True) == FLAG_NONFINITE
    assert st.flags() == 0


def test_diag_resnet18_full_size_trajectory(gpu_lib):
    """ResNet-18 at batch 128, 224x224 (11,679,912 weights), in the launch
    configuration the benchmark times: 100 free-running steps over two
    pre-drawn input batches (odd steps the first, even steps the second).
    Per layer, sampled output rows o and input columns j (the bias column
    included): dA[j] and dG[o] of both batches from the oracle's own columns,
    and the oracle's diagonal step run for 100 steps on those entries alone
    (the entries of a diagonal step do not interact), compared with the
    library's F, V and W after step 1 and step 100, and its dA, dG."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    cfg = synth.full_config("resnet18_diag")
    hp = synth.hparams(cfg)
    st = KfacStack(cfg.layers, "diag", pool=2)
    inputs = [[], []]
    for li in range(len(cfg.layers)):
        st.set_state(li, synth.initial_state(cfg, li))
    for slot in range(2):
        for li in range(len(cfg.layers)):
            inp = synth.step_inputs(cfg, slot + 1, li)
            st.set_inputs(li, inp, slot=slot)
            inputs[slot].append(inp)
        say(f"resnet18 full-size input batch {slot + 1} resident")
    rng = np.random.default_rng(123)
    samples = []
    for li, L in enumerate(cfg.layers):
        js = np.unique(np.concatenate([[0, L.d_a - 1], rng.integers(0, L.d_a, 6)]))
        os_ = np.unique(np.concatenate([[0, L.d_out - 1], rng.integers(0, L.d_out, 6)]))
        dA = [np.array([np.mean(oracle.activation_column(L, inputs[b][li]["a"], j) ** 2) for j in js]) for b in (0, 1)]
        dG = [np.array([np.mean(oracle.gradient_column(L, inputs[b][li]["g"], o) ** 2) for o in os_]) for b in (0, 1)]
        init = synth.initial_state(cfg, li)
        aug = lambda w, b: np.concatenate([w, b[:, None]], 1) if L.has_bias else w
        grads = [aug(inputs[b][li]["grad_w"], inputs[b][li]["grad_b"])[np.ix_(os_, js)] for b in (0, 1)]
        samples.append(dict(js=js, os=os_, dA=dA, dG=dG, grads=grads,
                            state={"w": aug(init["w"], init.get("b"))[np.ix_(os_, js)].astype(np.float64),
                                   "mom_w": np.zeros((len(os_), len(js))),
                                   "F_w": aug(init["F_w"], init.get("F_b"))[np.ix_(os_, js)].astype(np.float64)}))
    say("oracle entries of both batches ready")

    def oracle_step(smp, b):
        # the sampled entries as one bias-free linear layer with one row:
        # a = sqrt(dA), g = sqrt(dG) give the oracle's dG dA outer product
        one = synth.linear("entries", len(smp["js"]), len(smp["os"]), 1, bias=False)
        out, flags = oracle.step_diag(one, smp["state"], {"a": np.sqrt(smp["dA"][b])[None, :],
                                                          "g": np.sqrt(smp["dG"][b])[None, :],
                                                          "grad_w": smp["grads"][b]}, hp)
        assert flags == 0
        smp["state"] = {k: out[k] for k in ("w", "mom_w", "F_w")}

    def compare(step, b):
        worst = {}
        for li, (L, smp) in enumerate(zip(cfg.layers, samples)):
            got = st.get_state(li)
            aug = lambda w, bb: np.concatenate([w, bb[:, None]], 1) if L.has_bias else w
            sel = np.ix_(smp["os"], smp["js"])
            pairs = (("dA", got["dA"][smp["js"]], smp["dA"][b]), ("dG", got["dG"][smp["os"]], smp["dG"][b]),
                     ("F", aug(got["F_w"], got.get("F_b"))[sel], smp["state"]["F_w"]),
                     ("V", aug(got["mom_w"], got.get("mom_b"))[sel], smp["state"]["mom_w"]),
                     ("W", aug(got["w"], got.get("b"))[sel], smp["state"]["w"]))
            for k, x, y in pairs:
                e = max_rel(x, y)
                worst[k] = max(worst.get(k, 0.0), e)
                assert e <= 1e-4, (step, L.name, k, e)
        say(f"step {step}: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))

    H = st.hparams(hp)
    for t in range(1, 101):
        st.use_inputs((t - 1) % 2)
        st.step(H)
        for smp in samples:
            oracle_step(smp, (t - 1) % 2)
        if t in (1, 100):
            torch.cuda.synchronize()
            assert st.flags() == 0
            compare(t, (t - 1) % 2)


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_diag_degenerate_shapes_and_ema_limits(gpu_lib, beta):
    """1 -> 1 and single-row layers and a 1 x 1 single-channel conv at EMA
    decay 0 (F is this batch's dG dA) and 1 (F is kept)."""
    L = [synth.linear("one_one", 1, 1, 6, bias=True),
         synth.linear("one_row", 5, 4, 1, bias=True),
         synth.conv("pointwise", 1, 1, 1, 1, 0, 2, 3)]
    cfg = with_layers(synth.small_config("resnet18_diag"), L, steps=2, ema_decay=beta)
    lockstep(cfg, cfg.steps, TOL, DIAG_KEYS)


def test_diag_graph_replays_match_eager(gpu_lib):
    """One diagonal step (reduction, finish, parameter pass) captured in a HIP
    graph through torch.cuda.graph on ResNet-18 layer kinds; three replays,
    each followed by eager work and a synchronisation, match three eager
    steps on the same inputs bitwise."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    cfg = synth.small_config("resnet18_diag")
    H = KfacStack.hparams(synth.hparams(cfg))

    def make():
        st = KfacStack(cfg.layers, "diag")
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, 1, li))
        return st

    eager, graphed = make(), make()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(H)
    torch.cuda.synchronize()
    for rep in range(3):
        eager.step(H)
        g.replay()
        torch.cuda.synchronize()
        assert float(torch.ones(1000, device="cuda").sum().item()) == 1000.0   # eager work between replays
        assert graphed.flags() == 0 and eager.flags() == 0
        for li in range(len(cfg.layers)):
            a, b = eager.get_state(li), graphed.get_state(li)
            for k in a:
                assert np.array_equal(a[k], b[k]), (rep, cfg.layers[li].name, k)
    say("diagonal graph replays match eager steps bitwise")
