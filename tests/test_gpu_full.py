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


@pytest.mark.parametrize("packed", [False, True])
def test_single_workgroup_paths(gpu_lib, packed):
    """Steps whose layers all fit one 128-block take one workgroup per factor
    (factor SYRK and EMA), per factor (the whole inverse) and per layer
    (preconditioning and update).  Edge cases of those kernels: d = 128
    exactly (ten upper 32-blocks, three per wavefront), 300 rows (five 64-row
    chunks, the last partial: chunk pairs and an odd count), an odd row
    count in the last chunk (77 rows), exactly one chunk (64 rows), widths
    that are not multiples of 32, several factors and layers per launch,
    and packed factor storage."""
    L = [synth.linear("full_block", 127, 128, 300, bias=True),
         synth.linear("odd_rows", 33, 97, 77, bias=False),
         synth.linear("one_chunk", 5, 3, 64, bias=True)]
    cfg = with_layers(synth.full_config("fc64"), L, steps=3, act_std=1.0, grad_std=1e-2)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS, packed=packed)


def test_bias_column_layers(gpu_lib):
    """Biased layers whose d_in is a whole number of 128-wide tiles: the
    preconditioning GEMMs cover the weight columns and the bias column is two
    matrix-vector products (16-byte loads when d_out is a multiple of 4,
    scalar loads otherwise), beside a layer of the same kind without the
    split (d_in = 200)."""
    L = [synth.linear("vec", 256, 300, 900, bias=True),
         synth.linear("scalar", 384, 130, 700, bias=True),
         synth.linear("nosplit", 200, 128, 500, bias=True)]
    cfg = with_layers(synth.full_config("fc64"), L, steps=3, act_std=1.0, grad_std=1e-2)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_conv_split_k_and_layouts(gpu_lib):
    """Convolution factors (im2col rows and transposed gradients, then the
    row-major SYRK): a 7x7/2 stem with 16,900 rows (9 row splits summed by the
    reduce) and 147 unfold columns (a ragged 64-column im2col tile), a 3x3
    conv with 7 output channels (a ragged row pitch of 8), a strided conv with
    a bias column."""
    L = [synth.conv("stem", 3, 8, 7, 2, 3, 4, 130),
         synth.conv("odd_plane", 5, 7, 3, 1, 1, 3, 7),
         synth.conv("even_plane", 6, 9, 3, 2, 1, 2, 16, bias=True)]
    cfg = with_layers(synth.small_config("resnet50_kfac"), L, steps=2)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


@pytest.mark.parametrize("d_in", [150, 256])
def test_sgd_reduction_update_phase(gpu_lib, d_in):
    """UPDATE phase alone with identity inverses: the step is SGD with momentum
    and weight decay (closed form from the oracle's update); d_in = 256 takes
    the bias-column matrix-vector path."""
    import torch
    from second_order_optimizer_amd import PHASE_UPDATE
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.full_config("fc64"), [synth.linear("fc", d_in, 70, 8, bias=True)])
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


@pytest.mark.parametrize("d_in,d_out,bad", [(200, 140, 150), (100, 40, 50)])
def test_not_pd_keeps_inverse(gpu_lib, d_in, d_out, bad):
    """A factor with a negative eigenvalue (EMA decay 1 keeps it) fails the
    Cholesky: KFAC_FLAG_NOT_PD is raised and that inverse is left unchanged,
    while the positive definite G is still inverted; with multi-block factors
    and with factors of one diagonal block (the single-stream schedule)."""
    import torch
    from second_order_optimizer_amd import FLAG_NOT_PD, PHASE_FACTORS, PHASE_INVERT
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.full_config("fc64"), [synth.linear("fc", d_in, d_out, 16, bias=True)])
    L = cfg.layers[0]
    st = KfacStack(cfg.layers, "full")
    s0 = synth.initial_state(cfg, 0)
    A = np.eye(L.d_a, dtype=np.float32)
    A[bad, bad] = -10 * cfg.damping
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


def test_bf16_factor_row_chunks(gpu_lib):
    """A bf16 factor whose input spans more than 2 GiB (140,000 rows x 8,192
    columns) exceeds the 32-bit range of the direct-to-LDS loads: the SYRK
    runs it as two row chunks (the EMA on the first, beta = 1 on the second).
    FACTORS phase only; sampled entries of A, bias row included, vs the
    oracle's column products, 2e-2."""
    import torch
    from second_order_optimizer_amd import PHASE_FACTORS
    from second_order_optimizer_amd.stack import KfacStack
    L = synth.linear("wide", 8192, 64, 140000, bias=True)
    cfg = with_layers(synth.small_config("pair16k_bf16"), [L], steps=1)
    hp = synth.hparams(cfg)
    st = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype)
    st.set_state(0, synth.initial_state(cfg, 0))
    inp = synth.step_inputs(cfg, 1, 0)
    st.set_inputs(0, inp)
    say("row-chunk layer resident")
    st.step(st.hparams(hp, refresh=False, phase_mask=PHASE_FACTORS))
    torch.cuda.synchronize()
    assert st.flags() == 0
    got = st.get_state(0)["A"]
    eps = hp["ema_decay"]
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([[0, 8191, 8192], rng.integers(0, 8192, 5)]))
    cols = {j: oracle.activation_column(L, inp["a"], j) for j in idx}
    ref = np.array([[eps * (i == j) + (1 - eps) * cols[i] @ cols[j] / L.rows for j in idx] for i in idx])
    e = max_rel(got[np.ix_(idx, idx)], ref)
    say(f"row-chunk factor worst {e:.2e}")
    assert e <= 2e-2


@pytest.mark.parametrize("extra", [0, 24])
def test_graph_replays_match_eager(gpu_lib, extra):
    """One full step (factors; the two-level Cholesky with its far updates
    and the inverse assembly on the library's side streams; update)
    captured in a HIP graph through torch.cuda.graph on ResNet-50 layer kinds
    (factors of up to 9 Cholesky blocks, three outer panels) plus a biased
    256-input layer (its bias column on the side stream beside the update
    GEMMs), and with 24 more small layers (more problems than one launch's
    table holds: every GEMM kind in several launches); three replays, each
    followed by eager work and a synchronisation, match three eager steps on
    the same inputs bitwise."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    base = synth.small_config("resnet50_kfac")
    more = [synth.linear(f"small{i}", 48, 40, 16, bias=(i % 2 == 0)) for i in range(extra)]
    cfg = with_layers(base, list(base.layers) + [synth.linear("fc_split", 256, 96, 32, bias=True)] + more)
    H = KfacStack.hparams(synth.hparams(cfg), refresh=True)

    def make():
        st = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype)
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, 1, li))
        return st

    eager, graphed = make(), make()
    warm = make()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        warm.step(H)          # the capture stream's side streams and events exist before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
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
    say("graph replays match eager steps bitwise")


@pytest.mark.parametrize("ema", [0.0, 1.0])
def test_degenerate_shapes_and_ema_limits(gpu_lib, ema):
    """A 1 -> 1 layer with a bias (2 x 2 and 1 x 1 factors), a single-row
    layer (rank-one batch factor), a 3 -> 2 layer without a bias and a 1 x 1
    single-channel conv, at EMA decay 0 (the factor is this batch's alone and
    the old one is not read) and 1 (the factor is kept); inverse every step."""
    L = [synth.linear("one_one", 1, 1, 6, bias=True),
         synth.linear("one_row", 5, 4, 1, bias=True),
         synth.linear("tiny", 3, 2, 5, bias=False),
         synth.conv("pointwise", 1, 1, 1, 1, 0, 2, 3)]
    cfg = with_layers(synth.full_config("fc64"), L, steps=2, act_std=1.0, grad_std=1e-2, ema_decay=ema,
                      refresh_every=1)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_bf16_factor_xcd_runs(gpu_lib):
    """Ten bf16 layers 1024 -> 768 with a bias: one factor launch of 160
    tiles, whose first 128 go to the XCDs in runs of 16 consecutive tiles and
    the rest in order; every factor entry checked against the oracle."""
    L = synth.mlp_layers(5, 1024, 768, 64)
    cfg = with_layers(synth.small_config("mlp24_bf16"), L, steps=2, refresh_every=1)
    lockstep(cfg, cfg.steps, TOL16, FULL_KEYS)


def test_full_steps_from_two_threads(gpu_lib):
    """Two host threads each run three full steps (factors, inverse on the
    library's side streams, update) on their own stack and stream at the same
    time on one device; the results equal the same steps run one thread after
    the other, bitwise."""
    import threading
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    base = synth.small_config("resnet50_kfac")
    cfg = with_layers(base, list(base.layers) + [synth.linear("fc_split", 256, 96, 32, bias=True)])
    H = KfacStack.hparams(synth.hparams(cfg), refresh=True)

    def make(seed_step):
        st = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype)
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, seed_step, li))
        return st

    def run(st, stream):
        with torch.cuda.stream(stream):
            for _ in range(3):
                st.step(H, stream=stream)

    ref = [make(1), make(2)]
    s0 = torch.cuda.Stream()
    for st in ref:
        run(st, s0)
        torch.cuda.synchronize()
    par = [make(1), make(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    threads = [threading.Thread(target=run, args=(par[i], streams[i])) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for a_st, b_st in zip(ref, par):
        assert a_st.flags() == 0 and b_st.flags() == 0
        for li in range(len(cfg.layers)):
            a, b = a_st.get_state(li), b_st.get_state(li)
            for k in a:
                assert np.array_equal(a[k], b[k]), (cfg.layers[li].name, k)


def test_big_tile_gemms_lockstep(gpu_lib):
    """Nine biased fp32 layers 2048 -> 2048 at 64 rows: each preconditioning
    GEMM launch holds 9 x 64 = 576 tiles of 256 x 256, so it runs the
    256 x 256-tile kernels the large workloads time (the store epilogue, then
    the fused update), checked element by element against the oracle over
    three steps (inverse on steps 1 and 3)."""
    L = [synth.linear(f"wide{i}", 2048, 2048, 64, bias=True) for i in range(9)]
    cfg = with_layers(synth.full_config("fc64"), L, steps=3, act_std=1.0, grad_std=1e-2, refresh_every=2)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_big_tile_ragged_lockstep(gpu_lib):
    """Preconditioning launches of 576 256 x 256 tiles with ragged edges: 16
    layers 1040 -> 1008 with a bias (the bias column is not split off: the
    first product has 1041 columns and a contraction of 1040 + the bias index,
    over rows of the inverse that are not 16-byte aligned; the second product's
    rows 1008 end inside a tile) and 16 layers 1024 -> 1008 without one (rows
    of the inverse 16-byte aligned), three steps against the oracle."""
    L = []
    for i in range(16):
        L.append(synth.linear(f"odd{i}", 1040, 1008, 48, bias=True))
        L.append(synth.linear(f"even{i}", 1024, 1008, 48, bias=False))
    cfg = with_layers(synth.full_config("fc64"), L, steps=3, act_std=1.0, grad_std=1e-2, refresh_every=2)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_conv_factors_read_in_place(gpu_lib):
    """Convolution factors whose SYRK reads the NCHW tensor in place: the
    input of 1 x 1 stride-1 convolutions (8 x 8 and 16 x 16 planes, channel
    counts that end inside a tile) and the output gradients of 3 x 3
    convolutions with 16 x 16 output planes, at 1,024-4,096 rows (row splits),
    next to the same kinds that are laid out as rows first (a strided 1 x 1
    convolution, 10 x 10 planes); 3 steps against the oracle."""
    L = [synth.conv("pw8", 96, 130, 1, 1, 0, 16, 8),
         synth.conv("pw16", 64, 200, 1, 1, 0, 16, 16),
         synth.conv("c3", 40, 72, 3, 1, 1, 4, 16),
         synth.conv("c3s", 24, 64, 3, 2, 1, 4, 32),
         synth.conv("pw_s2", 48, 80, 1, 2, 0, 4, 16),
         synth.conv("pw10", 56, 90, 1, 1, 0, 8, 10)]
    cfg = with_layers(synth.small_config("resnet50_kfac"), L, steps=3)
    lockstep(cfg, cfg.steps, TOL32, FULL_KEYS)


def test_full_nonfinite_flag(gpu_lib):
    """A NaN in the weight gradient of a layer whose update runs in the GEMM
    epilogue, and separately in the bias gradient of a layer whose bias
    column runs as matrix-vector products, each raise KFAC_FLAG_NONFINITE;
    reading with clear resets the flag word."""
    import torch
    from second_order_optimizer_amd import FLAG_NONFINITE
    from second_order_optimizer_amd.stack import KfacStack
    L = [synth.linear("gemm", 100, 40, 16, bias=True), synth.linear("bias_split", 128, 40, 16, bias=True)]
    cfg = with_layers(synth.full_config("fc64"), L, steps=1)
    for li, key, where in ((0, "grad_w", (3, 7)), (1, "grad_b", (5,))):
        st = KfacStack(cfg.layers, "full")
        for lj in range(2):
            st.set_state(lj, synth.initial_state(cfg, lj))
            inp = synth.step_inputs(cfg, 1, lj)
            if lj == li:
                inp[key] = inp[key].copy()
                inp[key][where] = np.nan
            st.set_inputs(lj, inp)
        st.step(st.hparams(synth.hparams(cfg), refresh=True))
        torch.cuda.synchronize()
        assert st.flags(clear=True) == FLAG_NONFINITE, key
        assert st.flags() == 0


@pytest.mark.parametrize("variant", ["full", "diag"])
def test_resume_from_copied_state(gpu_lib, variant):
    """Checkpoint / resume: after two steps the whole state (W, V and the
    factors and inverses, or F) is copied to the host and into a new stack
    with its own workspace; two more steps there equal two more steps of the
    uninterrupted stack, bit for bit."""
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    cfg = synth.small_config("resnet50_kfac" if variant == "full" else "resnet18_diag")
    hp = synth.hparams(cfg)
    n = len(cfg.layers)

    def steps(st, ts):
        for t in ts:
            for li in range(n):
                st.set_inputs(li, synth.step_inputs(cfg, t, li))
            refresh = synth.refresh_at(cfg, t) if variant == "full" else True
            st.step(st.hparams(hp, refresh=refresh))
        torch.cuda.synchronize()

    a = KfacStack(cfg.layers, variant)
    for li in range(n):
        a.set_state(li, synth.initial_state(cfg, li))
    steps(a, (1, 2))
    ckpt = [a.get_state(li) for li in range(n)]
    b = KfacStack(cfg.layers, variant)
    for li in range(n):
        b.set_state(li, ckpt[li])
    steps(a, (3, 4))
    steps(b, (3, 4))
    assert a.flags() == 0 and b.flags() == 0
    for li in range(n):
        x, y = a.get_state(li), b.get_state(li)
        for k in x:
            assert np.array_equal(x[k], y[k]), (cfg.layers[li].name, k)


def test_capture_beside_steps_on_other_streams(gpu_lib):
    """Thread A captures a full step (with the Cholesky side streams) into a
    graph on its stream; while the capture is open, thread B runs three full
    steps on another stream.  B's results equal the same steps run alone, and
    three replays of A's graph equal three eager steps, bit for bit."""
    import threading
    import torch
    from second_order_optimizer_amd.stack import KfacStack
    base = synth.small_config("resnet50_kfac")
    cfg = with_layers(base, list(base.layers) + [synth.linear("fc_split", 256, 96, 32, bias=True)])
    H = KfacStack.hparams(synth.hparams(cfg), refresh=True)

    def make(t):
        st = KfacStack(cfg.layers, "full", cfg.act_dtype, cfg.grad_dtype)
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            st.set_inputs(li, synth.step_inputs(cfg, t, li))
        return st

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    warm = make(1)
    for s in (sa, sb):
        with torch.cuda.stream(s):
            warm.step(H, stream=s)     # side streams of both streams exist before the capture
    torch.cuda.synchronize()
    ref_b = make(2)
    with torch.cuda.stream(sb):
        for _ in range(3):
            ref_b.step(H, stream=sb)
    eager_a, graphed, par_b = make(1), make(1), make(2)
    torch.cuda.synchronize()
    captured, b_done, errors = threading.Event(), threading.Event(), []

    def thread_a():
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=sa, capture_error_mode="thread_local"):
                graphed.step(H)
                captured.set()
                if not b_done.wait(timeout=60):
                    raise RuntimeError("thread B did not finish")
            thread_a.graph = g
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)
            captured.set()

    def thread_b():
        try:
            captured.wait(timeout=60)
            for _ in range(3):
                par_b.step(H, stream=sb)
        except Exception as e:  # noqa: BLE001
            errors.append(e)
        finally:
            b_done.set()

    ta, tb = threading.Thread(target=thread_a), threading.Thread(target=thread_b)
    ta.start(); tb.start(); ta.join(); tb.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for li in range(len(cfg.layers)):
        x, y = ref_b.get_state(li), par_b.get_state(li)
        for k in x:
            assert np.array_equal(x[k], y[k]), ("B", cfg.layers[li].name, k)
    for rep in range(3):
        eager_a.step(H)
        thread_a.graph.replay()
        torch.cuda.synchronize()
        for li in range(len(cfg.layers)):
            x, y = eager_a.get_state(li), graphed.get_state(li)
            for k in x:
                assert np.array_equal(x[k], y[k]), ("A", rep, cfg.layers[li].name, k)
    assert eager_a.flags() == 0 and graphed.flags() == 0 and par_b.flags() == 0
