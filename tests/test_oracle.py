"""The oracle against its pins (CPU only), and planted mistakes in a private
copy of the oracle that the pins must catch."""
import importlib.util
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from tests import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kfac.py")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin(oracle)


def _fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mut_unfold_order(M):
    orig = M.unfold

    def unfold(x, k, stride, pad):
        U = orig(x, k, stride, pad)
        C = x.shape[1]
        return U.reshape(U.shape[0], C, k, k).transpose(0, 2, 3, 1).reshape(U.shape[0], -1)
    M.unfold = unfold


def _mut_unfold_no_pad_shift(M):
    orig = M.unfold
    M.unfold = lambda x, k, stride, pad: orig(np.roll(x, 1, axis=3), k, stride, pad)


def _mut_factor_norm(M):
    M.kronecker_factor = lambda rows: np.asarray(rows, np.float64).T @ np.asarray(rows, np.float64) / (len(rows) + 1)


def _mut_factor_transpose(M):
    M.kronecker_factor = lambda rows: np.asarray(rows, np.float64) @ np.asarray(rows, np.float64).T / len(rows)


def _mut_ema_swap(M):
    M.ema = lambda old, new, decay: (1 - decay) * np.asarray(old, np.float64) + decay * np.asarray(new, np.float64)


def _mut_inverse_no_damping(M):
    orig = M.damped_inverse
    M.damped_inverse = lambda F, damping: orig(F, 0.0) if damping < 0.2 else orig(F, damping)


def _mut_inverse_wrong_product(M):
    def damped_inverse(F, damping):
        L = np.linalg.cholesky(np.asarray(F, np.float64) + damping * np.eye(len(F)))
        Z = scipy.linalg.solve_triangular(L, np.eye(len(F)), lower=True)
        return Z @ Z.T
    M.damped_inverse = damped_inverse


def _mut_precond_drop_A(M):
    M.precondition = lambda Gi, g, Ai: np.asarray(Gi) @ np.asarray(g)


def _mut_precond_squared(M):
    M.precondition = lambda Gi, g, Ai: np.asarray(Gi) @ np.asarray(g) @ np.asarray(Ai) @ np.asarray(Ai)


def _mut_wd_sign(M):
    orig = M.momentum_update
    M.momentum_update = lambda w, v, p, lr, mu, wd: orig(w, v, p, lr, mu, -wd)


def _mut_dampening(M):
    def momentum_update(w, v, p, lr, mu, wd):
        d = np.asarray(p) + wd * np.asarray(w)
        v2 = mu * np.asarray(v) + (1 - mu) * d
        return np.asarray(w) - lr * v2, v2
    M.momentum_update = momentum_update


def _mut_nesterov(M):
    def momentum_update(w, v, p, lr, mu, wd):
        d = np.asarray(p) + wd * np.asarray(w)
        v2 = mu * np.asarray(v) + d
        return np.asarray(w) - lr * (d + mu * v2), v2
    M.momentum_update = momentum_update


def _mut_bias_first(M):
    orig = M.layer_rows

    def layer_rows(layer, a, g):
        ab, gr = orig(layer, a, g)
        if layer.has_bias:
            ab = np.concatenate([ab[:, -1:], ab[:, :-1]], axis=1)
        return ab, gr
    M.layer_rows = layer_rows


def _mut_diag_abs(M):
    def diag_factors(layer, a, g):
        ab, gr = M.layer_rows(layer, a, g)
        return np.abs(ab).mean(axis=0) ** 2, (gr * gr).mean(axis=0)
    M.diag_factors = diag_factors


def _mut_widen_low_half(M):
    M.widen = lambda x: (np.asarray(x).astype(np.uint32).view(np.float32).astype(np.float64)
                         if np.asarray(x).dtype == np.uint16 else np.asarray(x).astype(np.float64))


def _mut_unfold_column_kh_kw(M):
    def unfold_column(x, k, stride, pad, j):
        c, kw, kh = j // (k * k), (j // k) % k, j % k     # kernel row and column swapped
        return M.unfold_column.__wrapped__(x, k, stride, pad, (c * k + kh) * k + kw)
    unfold_column.__wrapped__ = M.unfold_column
    M.unfold_column = unfold_column


def _mut_gradient_column_order(M):
    orig = M.gradient_column

    def gradient_column(layer, g, o):
        if layer.kind == "conv":
            return M.widen(np.asarray(g)[:, o].transpose(0, 2, 1)).reshape(-1)   # positions column-major
        return orig(layer, g, o)
    M.gradient_column = gradient_column


def _mut_activation_column_bias(M):
    orig = M.activation_column

    def activation_column(layer, a, j):
        col = orig(layer, a, j)
        return col * 0.0 if (layer.has_bias and j == layer.d_in) else col
    M.activation_column = activation_column


def _mut_bn_fisher_per_element(M):
    def bn_fisher(xhat, g):
        x, gg = M.widen(xhat), M.widen(g)
        return ((gg * x) ** 2).sum(axis=(2, 3)).mean(axis=0), (gg ** 2).sum(axis=(2, 3)).mean(axis=0)
    M.bn_fisher = bn_fisher


def _mut_bn_layer_damping(M):
    orig = M.step_bn
    M.step_bn = lambda layer, state, inputs, hp: orig(layer, state, inputs, dict(hp, damping_bn=hp["damping"]))


def _mut_rescale_d_in(M):
    M.rescale_weights = lambda w, d_out, eps: (np.asarray(w, np.float64) * np.sqrt(2.0 * np.shape(w)[1]) /
                                                (np.linalg.norm(w) + eps))


def _mut_schedule_off_by_one(M):
    orig = M.schedule
    M.schedule = lambda s, t: orig(s, t + 1)


def _mut_pack_by_columns(M):
    M.pack_upper = lambda A: np.concatenate([np.asarray(A)[:j + 1, j] for j in range(np.shape(A)[0])])


MUTANTS = [_mut_unfold_order, _mut_unfold_no_pad_shift, _mut_factor_norm, _mut_factor_transpose,
           _mut_ema_swap, _mut_inverse_no_damping, _mut_inverse_wrong_product, _mut_precond_drop_A,
           _mut_precond_squared, _mut_wd_sign, _mut_dampening, _mut_nesterov, _mut_bias_first,
           _mut_diag_abs, _mut_widen_low_half, _mut_unfold_column_kh_kw,
           _mut_gradient_column_order, _mut_activation_column_bias, _mut_bn_fisher_per_element,
           _mut_bn_layer_damping, _mut_rescale_d_in, _mut_schedule_off_by_one, _mut_pack_by_columns]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutate):
    M = _fresh_oracle()
    mutate(M)
    caught = []
    for pin in P.ALL_PINS:
        try:
            ok = pin(M)
        except Exception:
            ok = False
        if not ok:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutate.__name__}"


def test_oracle_has_no_product_imports():
    """The oracle imports nothing from the HIP path or its binding."""
    for fn in os.listdir(os.path.dirname(ORACLE_SRC)):
        if fn.endswith(".py"):
            src = open(os.path.join(os.path.dirname(ORACLE_SRC), fn)).read()
            assert "second_order_optimizer_amd" not in src
            assert "import synth" not in src and "from synth" not in src
