"""Float64 CPU oracle of the K-FAC optimizer step -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import or call anything here.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

See ``oracle.kfac`` for the passages each function follows and for the
readings taken where the pages are silent.
"""
from .kfac import (  # noqa: F401
    FLAG_NOT_PD,
    FLAG_NONFINITE,
    widen,
    unfold,
    unfold_column,
    activation_column,
    gradient_column,
    layer_rows,
    kronecker_factor,
    ema,
    damped_inverse,
    precondition,
    momentum_update,
    diag_factors,
    step_full,
    step_diag,
    step_bn,
    bn_fisher,
    rescale_weights,
    schedule,
    pack_upper,
    unpack_upper,
    aug_weight,
    split_weight,
)
