"""kfac_step_diag_noalloc (C ABI): the diagonal step without a workspace,
with its scratch in the library's own device array, against kfac_step_diag
on the same state and inputs."""
import numpy as np
import pytest

import synth
from tests.parity import say, with_layers

pytestmark = pytest.mark.gpu


def _stacks(cfg, t=1, nan_at=None):
    from second_order_optimizer_amd.stack import KfacStack
    pair = []
    for _ in range(2):
        st = KfacStack(cfg.layers, "diag")
        for li in range(len(cfg.layers)):
            st.set_state(li, synth.initial_state(cfg, li))
            inp = synth.step_inputs(cfg, t, li)
            if nan_at is not None and li == 0:
                inp["grad_w"] = inp["grad_w"].copy()
                inp["grad_w"][nan_at] = np.nan
            st.set_inputs(li, inp)
        pair.append(st)
    return pair


def test_noalloc_matches_workspace_step(gpu_lib):
    """Two calls in a row on one GPU, the second on a smaller stack: ResNet-18
    layer kinds (batch 4 at 64x64: conv window sums through the scratch), then
    a conv and a linear layer with 700 rows (chunk partials through the
    scratch); every tensor equals kfac_step_diag's, bit for bit, and the
    caller's flag word stays clear."""
    import torch
    import second_order_optimizer_amd as K
    big = synth.small_config("resnet18_diag")
    small = with_layers(big, [synth.conv("c", 3, 8, 3, 2, 1, 2, 9), synth.linear("fc", 20, 6, 700, bias=True)],
                        steps=1)
    flags = torch.zeros(64, dtype=torch.int32, device="cuda")
    for cfg in (big, small):
        ref, new = _stacks(cfg)
        H = ref.hparams(synth.hparams(cfg))
        ref.step(H)
        K.step_diag_noalloc(new.desc, H, flags.data_ptr())
        torch.cuda.synchronize()
        for li, L in enumerate(cfg.layers):
            a, b = ref.get_state(li), new.get_state(li)
            for k in a:
                assert np.array_equal(a[k], b[k]), (cfg.name, L.name, k)
        assert K.read_flags(flags.data_ptr()) == 0 and ref.flags() == 0
        say(f"no-alloc step matches the workspace step on {len(cfg.layers)} layers")


def test_noalloc_flags_and_size_limit(gpu_lib):
    """A NaN gradient raises KFAC_FLAG_NONFINITE in the caller's flag word
    (cleared by kfac_read_flags); a stack whose scratch exceeds 32 MiB (a
    3 x 2048 x 2048 input plane: 48 MiB of sums) is rejected with
    KFAC_ERR_WORKSPACE before anything runs (its parameters are unchanged)."""
    import torch
    import second_order_optimizer_amd as K
    from second_order_optimizer_amd.stack import KfacStack
    cfg = with_layers(synth.small_config("resnet18_diag"), [synth.linear("fc", 16, 8, 4)], steps=1)
    _, st = _stacks(cfg, nan_at=(3, 5))
    flags = torch.zeros(64, dtype=torch.int32, device="cuda")
    K.step_diag_noalloc(st.desc, st.hparams(synth.hparams(cfg)), flags.data_ptr())
    torch.cuda.synchronize()
    assert K.read_flags(flags.data_ptr(), clear=True) == K.FLAG_NONFINITE
    assert K.read_flags(flags.data_ptr()) == 0
    huge = with_layers(cfg, [synth.conv("huge", 3, 2, 3, 2, 1, 1, 2048)], steps=1)
    assert K.workspace_size(KfacStack(huge.layers, "diag").desc, K.MODE_DIAG) > K.NOALLOC_SCRATCH_BYTES
    hs = KfacStack(huge.layers, "diag")
    hs.set_state(0, synth.initial_state(huge, 0))
    before = hs.get_state(0)
    with pytest.raises(K.KfacError) as e:
        K.step_diag_noalloc(hs.desc, hs.hparams(synth.hparams(huge)), flags.data_ptr())
    assert e.value.status == K.KFAC_ERR_WORKSPACE
    torch.cuda.synchronize()
    after = hs.get_state(0)
    for k in before:
        assert np.array_equal(before[k], after[k]), k
