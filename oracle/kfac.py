"""Float64 CPU oracle of the K-FAC optimizer step -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may use this module.  It is written from the pages' description of the
method, plainly and slowly, in float64; it shares no code with the HIP path.

Sources (the pages' titles; sections as headed there):
  [KFAC]  Osawa et al., "Large-Scale Distributed Second-Order Optimization
          Using Kronecker-Factored Approximate Curvature for Deep
          Convolutional Neural Networks" (arXiv 1811.12019v5 summary):
          section 3.2 (K-FAC: layer-wise Kronecker factors built from
          activations and output gradients; the FIM inverse through the
          factor inverses), section 3.4 (symmetric factors), section 4.2
          (damping), section 4.3 (momentum), sections 1 and 5.4 (inverse
          refreshed less often than every step).
  [CAFIN] "CAFIN: CUDA-accelerated Adaptive Fisher Information Matrix Network
          Optimization via GPU-Native Kernel Fusion" (briefing): Introduction
          (AdaFisher's diagonal Kronecker FIM with exponential moving
          averages) and "Kernel Fusion Strategy" (the per-step order: load
          gradient and parameters, update the FIM EMA, precondition, apply
          momentum and weight decay, write the parameters in place).

Readings taken where the pages leave a step open (each is stated once more
where it is used):
  R1  factors are normalised by the number of rows N (batch rows for a
      linear layer, batch x output positions for a convolution);
  R2  a layer with a bias gets a constant-1 column appended last to its
      activations, and its weight is augmented as [W | b];
  R3  convolution inputs are unfolded with zero padding, columns in
      (channel, kernel row, kernel column) order;
  R5  Tikhonov damping on each factor with the same lambda: (A + lambda I)^-1,
      (G + lambda I)^-1;
  R6  step t refreshes the inverses when the caller asks for it; the factor
      EMA of step t happens before that step's inversion;
  R7  weight decay is added after preconditioning: D = P + wd * W;
  R8  heavy-ball momentum without dampening: V = mu V + D, W = W - lr V;
  R9  diagonal variant: EMA of the per-parameter product dG[o] * dA[j],
      preconditioner 1 / (F + lambda), no square root, no bias correction;
  R17 batch normalisation [KFAC sections 1 and 5.4: its Fisher approximated
      as diagonal]: the diagonal of the Fisher of gamma and beta from
      per-sample gradients, mean over samples of (sum_hw g x_hat)^2 and of
      (sum_hw g)^2, with the same EMA / damping / momentum tail (damping
      scaled for batch-norm layers, section 4.2);
  R18 weight rescaling [KFAC section 4.4]: after the update the layer's
      weight (bias excluded) is scaled to Frobenius norm sqrt(2 d_out), the
      norm of a He-initialised d_out x d_in weight; epsilon in the divisor;
  R19 warm-up damping [KFAC section 4.2]: from gamma(0) to gamma_target over
      t_warmup steps, linearly (or geometrically), then constant;
  R20 refresh schedule [KFAC sections 1 and 5.4]: both inverses every step
      for the first steps, then A and G on their own intervals;
  R21 packed factor storage [KFAC section 3.4]: the upper triangle, row by
      row, d (d + 1) / 2 entries.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

FLAG_NOT_PD = 1      # a damped factor was not positive definite: its inverse is kept
FLAG_NONFINITE = 2   # a non-finite value reached the parameters


# ---------------------------------------------------------------------------
# inputs

def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 copy of a float32 array or of bfloat16 bit patterns
    (uint16): a bfloat16 is the upper half of a float32."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def unfold(x: np.ndarray, k: int, stride: int, pad: int) -> np.ndarray:
    """im2col of an NCHW input (reading R3).

    Row n = (b * H_out + ho) * W_out + wo, column j = (c * k + kh) * k + kw,
    U[n, j] = x[b, c, ho*stride - pad + kh, wo*stride - pad + kw], zero
    outside the image.  A convolution layer's A factor is built from these
    rows [KFAC section 3.2; Kronecker factors of convolutions]."""
    B, C, H, W = x.shape
    Ho = (H + 2 * pad - k) // stride + 1
    Wo = (W + 2 * pad - k) // stride + 1
    xp = np.zeros((B, C, H + 2 * pad, W + 2 * pad), np.float64)
    xp[:, :, pad:pad + H, pad:pad + W] = x
    U = np.empty((B, Ho, Wo, C, k, k), np.float64)
    for kh in range(k):
        for kw in range(k):
            win = xp[:, :, kh:kh + stride * (Ho - 1) + 1:stride, kw:kw + stride * (Wo - 1) + 1:stride]
            U[:, :, :, :, kh, kw] = win.transpose(0, 2, 3, 1)
    return U.reshape(B * Ho * Wo, C * k * k)


def unfold_column(x: np.ndarray, k: int, stride: int, pad: int, j: int) -> np.ndarray:
    """Column j of ``unfold(x, k, stride, pad)`` alone (same definition, for
    checking single outputs of full-size inputs): j = (c * k + kh) * k + kw."""
    B, C, H, W = x.shape
    c, kh, kw = j // (k * k), (j // k) % k, j % k
    Ho = (H + 2 * pad - k) // stride + 1
    Wo = (W + 2 * pad - k) // stride + 1
    hi = np.arange(Ho) * stride - pad + kh          # input row of each output row
    wi = np.arange(Wo) * stride - pad + kw
    hv, wv = (hi >= 0) & (hi < H), (wi >= 0) & (wi < W)
    col = np.zeros((B, Ho, Wo))                     # zero where the tap is in the padding
    col[np.ix_(np.arange(B), np.flatnonzero(hv), np.flatnonzero(wv))] = widen(x[:, c][:, hi[hv]][:, :, wi[wv]])
    return col.reshape(-1)


def activation_column(layer, a: np.ndarray, j: int) -> np.ndarray:
    """Column j of a_bar (R1-R3) without building the whole matrix."""
    if layer.has_bias and j == layer.d_in:
        if layer.kind == "conv":
            B, C, H, W = a.shape
            n = B * ((H + 2 * layer.pad - layer.k) // layer.stride + 1) * ((W + 2 * layer.pad - layer.k) // layer.stride + 1)
        else:
            n = a.shape[0]
        return np.ones(n)
    if layer.kind == "conv":
        return unfold_column(a, layer.k, layer.stride, layer.pad, j)
    return widen(a[:, j])


def gradient_column(layer, g: np.ndarray, o: int) -> np.ndarray:
    """Column o of the output-gradient rows (conv: all samples and positions)."""
    if layer.kind == "conv":
        return widen(g[:, o]).reshape(-1)
    return widen(g[:, o])


def layer_rows(layer, a: np.ndarray, g: np.ndarray):
    """The rows the factors are built from: (a_bar [N, d_a], g [N, d_out]).

    ``layer`` needs ``kind`` ("linear" | "conv"), ``has_bias`` and, for a
    convolution, ``k``, ``stride``, ``pad``.  Linear: a [N, d_in], g [N, d_out].
    Convolution: a = x [B, C, H, W], g [B, C_out, H_out, W_out]; rows are
    (sample, output position) pairs in the unfold's order (R1, R3).  With a
    bias, a_bar = [a | 1] (R2)."""
    a = widen(a)
    g = widen(g)
    if layer.kind == "conv":
        a = unfold(a, layer.k, layer.stride, layer.pad)
        g = g.transpose(0, 2, 3, 1).reshape(-1, g.shape[1])
    if layer.has_bias:
        a = np.concatenate([a, np.ones((a.shape[0], 1))], axis=1)
    return a, g


# ---------------------------------------------------------------------------
# the step's pieces

def kronecker_factor(rows: np.ndarray) -> np.ndarray:
    """One batch's Kronecker factor: rows^T rows / N [KFAC section 3.2, R1].
    For activations this is the input factor A-hat, for output gradients the
    gradient factor G-hat."""
    rows = np.asarray(rows, np.float64)
    return rows.T @ rows / rows.shape[0]


def ema(old: np.ndarray, new: np.ndarray, decay: float) -> np.ndarray:
    """Exponential moving average [CAFIN Introduction]: decay*old + (1-decay)*new."""
    return decay * np.asarray(old, np.float64) + (1.0 - decay) * np.asarray(new, np.float64)


def damped_inverse(F: np.ndarray, damping: float) -> np.ndarray:
    """(F + damping I)^-1 through a Cholesky factorisation [KFAC sections 3.2
    and 4.2, R5]: F + damping I = L L^T, Z = L^-1 (triangular solve against I),
    inverse = Z^T Z.  Raises numpy.linalg.LinAlgError when F + damping I is not
    positive definite."""
    F = np.asarray(F, np.float64)
    d = F.shape[0]
    M = F + damping * np.eye(d)
    L = np.linalg.cholesky(M)
    Z = scipy.linalg.solve_triangular(L, np.eye(d), lower=True)
    return Z.T @ Z


def precondition(G_inv: np.ndarray, grad: np.ndarray, A_inv: np.ndarray) -> np.ndarray:
    """Natural-gradient direction for one layer: G_inv . grad . A_inv
    [KFAC section 3.2: the Kronecker-factored FIM is inverted through its
    factors; with row-major vec, (G kron A)^-1 vec(grad) = vec(G^-1 grad A^-1)]."""
    return np.asarray(G_inv, np.float64) @ np.asarray(grad, np.float64) @ np.asarray(A_inv, np.float64)


def momentum_update(w, v, p, lr: float, momentum: float, weight_decay: float):
    """Optimizer tail [CAFIN Kernel Fusion Strategy; KFAC section 4.3, R7, R8]:
    D = P + wd*W, V' = mu*V + D, W' = W - lr*V'.  Returns (W', V')."""
    w = np.asarray(w, np.float64)
    d = np.asarray(p, np.float64) + weight_decay * w
    v_new = momentum * np.asarray(v, np.float64) + d
    return w - lr * v_new, v_new


def diag_factors(layer, a: np.ndarray, g: np.ndarray):
    """Diagonal Kronecker factors [CAFIN Introduction, R9]:
    dA[j] = (1/N) sum_n a_bar[n, j]^2,  dG[o] = (1/N) sum_n g[n, o]^2."""
    abar, grows = layer_rows(layer, a, g)
    return (abar * abar).mean(axis=0), (grows * grows).mean(axis=0)


def aug_weight(w, b=None) -> np.ndarray:
    """[W | b] as float64 (R2); W may be a conv weight [C_out, C_in, k, k]."""
    w = np.asarray(w, np.float64).reshape(np.shape(w)[0], -1)
    if b is None:
        return w
    return np.concatenate([w, np.asarray(b, np.float64).reshape(-1, 1)], axis=1)


def split_weight(wa: np.ndarray, has_bias: bool):
    if has_bias:
        return wa[:, :-1], wa[:, -1]
    return wa, None


def bn_fisher(xhat: np.ndarray, g: np.ndarray):
    """Diagonal Fisher of a batch-norm layer's affine parameters [KFAC
    sections 1 and 5.4, R17].  With y = gamma x_hat + beta per channel, sample
    b's gradients are dgamma_b[c] = sum_hw g[b, c] x_hat[b, c] and
    dbeta_b[c] = sum_hw g[b, c]; the Fisher diagonal is their mean square over
    the samples.  xhat, g: [B, C, H, W].  Returns (f_gamma [C], f_beta [C])."""
    xhat = widen(xhat)
    g = widen(g)
    dgamma = (g * xhat).sum(axis=(2, 3))      # [B, C]
    dbeta = g.sum(axis=(2, 3))
    return (dgamma * dgamma).mean(axis=0), (dbeta * dbeta).mean(axis=0)


def rescale_weights(w: np.ndarray, d_out: int, eps: float) -> np.ndarray:
    """Weight rescaling after the update [KFAC section 4.4, R18]:
    W sqrt(2 d_out) / (||W||_F + eps)."""
    w = np.asarray(w, np.float64)
    return w * (np.sqrt(2.0 * d_out) / (np.linalg.norm(w) + eps))


def schedule(sched: dict, t: int):
    """Per-step damping and refresh choice [KFAC section 4.2 (R19), sections 1
    and 5.4 (R20)] for step t >= 1.  ``sched`` keys: damping_init,
    damping_target, warmup_steps, warmup_shape ("linear" | "geometric"),
    bn_damping_scale, dense_steps, refresh_every_a, refresh_every_g.
    Returns (damping, damping_bn, refresh_A, refresh_G)."""
    g0, gt, tw = sched["damping_init"], sched["damping_target"], sched["warmup_steps"]
    u = 1.0 if tw == 0 else min(t - 1, tw) / tw
    if sched["warmup_shape"] == "linear":
        lam = g0 + (gt - g0) * u
    else:
        lam = g0 * (gt / g0) ** u
    D = max(sched["dense_steps"], 1)
    ra = t <= D or (t - D) % sched["refresh_every_a"] == 0
    rg = t <= D or (t - D) % sched["refresh_every_g"] == 0
    return lam, sched["bn_damping_scale"] * lam, ra, rg


def pack_upper(M: np.ndarray) -> np.ndarray:
    """Packed storage of a symmetric factor [KFAC section 3.4, R21]: the upper
    triangle, row after row (row i contributes M[i, i:])."""
    M = np.asarray(M)
    return np.concatenate([M[i, i:] for i in range(M.shape[0])])


def unpack_upper(p: np.ndarray, d: int) -> np.ndarray:
    """The symmetric d x d matrix whose packed upper triangle is p."""
    p = np.asarray(p)
    M = np.zeros((d, d), p.dtype)
    k = 0
    for i in range(d):
        M[i, i:] = p[k:k + d - i]
        k += d - i
    return M + np.triu(M, 1).T


# ---------------------------------------------------------------------------
# whole steps

def step_full(layer, state: dict, inputs: dict, hp: dict, refresh):
    """One full K-FAC step for one layer, in the order the pages give
    [KFAC section 3.2; CAFIN Kernel Fusion Strategy]:

      1. rows a_bar, g of this batch (R1-R3);
      2. A <- ema(A, a_bar^T a_bar / N), G <- ema(G, g^T g / N);
      3. on a refresh step: A_inv = (A + lambda I)^-1, G_inv = (G + lambda I)^-1
         (R5, R6); ``refresh`` is a bool (both) or a pair (A, G) (R20); a
         factor that is not positive definite keeps its previous inverse and
         raises FLAG_NOT_PD;
      4. P = G_inv . grad_W_aug . A_inv;
      5. D = P + wd W_aug; V <- mu V + D; W_aug <- W_aug - lr V (R7, R8);
      6. with hp["rescale"], W <- rescale_weights(W) (R18).

    A batch-norm layer (kind "bn") takes the diagonal step of step_bn instead
    (R17).  ``state`` holds w, mom_w, A, G, A_inv, G_inv (+ b, mom_b with a
    bias); ``inputs`` holds a, g, grad_w (+ grad_b).  Returns (new_state,
    flags), new arrays in float64."""
    if layer.kind == "bn":
        return step_bn(layer, state, inputs, hp)
    ref_a, ref_g = (refresh, refresh) if isinstance(refresh, (bool, np.bool_, int)) else refresh
    eps, lam = hp["ema_decay"], hp["damping"]
    abar, grows = layer_rows(layer, inputs["a"], inputs["g"])
    A = ema(state["A"], kronecker_factor(abar), eps)
    G = ema(state["G"], kronecker_factor(grows), eps)
    A_inv = np.asarray(state["A_inv"], np.float64)
    G_inv = np.asarray(state["G_inv"], np.float64)
    flags = 0
    if ref_a:
        try:
            A_inv = damped_inverse(A, lam)
        except np.linalg.LinAlgError:
            flags |= FLAG_NOT_PD
    if ref_g:
        try:
            G_inv = damped_inverse(G, lam)
        except np.linalg.LinAlgError:
            flags |= FLAG_NOT_PD
    has_bias = layer.has_bias
    grad = aug_weight(inputs["grad_w"], inputs.get("grad_b") if has_bias else None)
    W = aug_weight(state["w"], state.get("b") if has_bias else None)
    V = aug_weight(state["mom_w"], state.get("mom_b") if has_bias else None)
    P = precondition(G_inv, grad, A_inv)
    W, V = momentum_update(W, V, P, hp["lr"], hp["momentum"], hp["weight_decay"])
    if not (np.all(np.isfinite(W)) and np.all(np.isfinite(V))):
        flags |= FLAG_NONFINITE
    w, b = split_weight(W, has_bias)
    mw, mb = split_weight(V, has_bias)
    if hp.get("rescale"):
        w = rescale_weights(w, np.shape(state["w"])[0], hp["rescale_eps"])
    out = {"A": A, "G": G, "A_inv": A_inv, "G_inv": G_inv, "P": P,
           "w": w.reshape(np.shape(state["w"])), "mom_w": mw.reshape(np.shape(state["w"]))}
    if has_bias:
        out["b"], out["mom_b"] = b, mb
    return out, flags


def _diagonal_tail(layer, state: dict, inputs: dict, hp: dict, target: np.ndarray, lam: float):
    """The elementwise part of a diagonal step [CAFIN Kernel Fusion Strategy,
    R7-R9]: F <- beta F + (1 - beta) target (per parameter, [W | b] layout);
    P = grad_W_aug / (F + lambda); D = P + wd W_aug; V <- mu V + D;
    W_aug <- W_aug - lr V.  Returns (out, flags) with w, mom_w, F_w (+ b,
    mom_b, F_b)."""
    has_bias = layer.has_bias
    F = aug_weight(state["F_w"], state.get("F_b") if has_bias else None)
    F = ema(F, target, hp["ema_decay"])
    grad = aug_weight(inputs["grad_w"], inputs.get("grad_b") if has_bias else None)
    W = aug_weight(state["w"], state.get("b") if has_bias else None)
    V = aug_weight(state["mom_w"], state.get("mom_b") if has_bias else None)
    P = grad / (F + lam)
    W, V = momentum_update(W, V, P, hp["lr"], hp["momentum"], hp["weight_decay"])
    flags = 0 if (np.all(np.isfinite(W)) and np.all(np.isfinite(V))) else FLAG_NONFINITE
    shape = np.shape(state["w"])
    w, b = split_weight(W, has_bias)
    mw, mb = split_weight(V, has_bias)
    fw, fb = split_weight(F, has_bias)
    out = {"P": P, "w": w.reshape(shape), "mom_w": mw.reshape(shape), "F_w": fw.reshape(shape)}
    if has_bias:
        out["b"], out["mom_b"], out["F_b"] = b, mb, fb
    return out, flags


def step_diag(layer, state: dict, inputs: dict, hp: dict):
    """One AdaFisher-style diagonal step for one layer [CAFIN Introduction and
    Kernel Fusion Strategy, R9]:

      1. dA, dG from this batch;
      2. F <- beta F + (1 - beta) dG[o] dA[j]   (per parameter, [W | b] layout);
      3. P = grad_W_aug / (F + lambda);
      4. D = P + wd W_aug; V <- mu V + D; W_aug <- W_aug - lr V;
      5. with hp["rescale"], W <- rescale_weights(W) (R18).

    A batch-norm layer (kind "bn") takes step_bn.  ``state`` holds w, mom_w,
    F_w (+ b, mom_b, F_b).  Returns (new_state, flags) with dA, dG included."""
    if layer.kind == "bn":
        return step_bn(layer, state, inputs, hp)
    dA, dG = diag_factors(layer, inputs["a"], inputs["g"])
    out, flags = _diagonal_tail(layer, state, inputs, hp, np.outer(dG, dA), hp["damping"])
    if hp.get("rescale"):
        out["w"] = rescale_weights(out["w"], np.shape(state["w"])[0], hp["rescale_eps"])
    out["dA"], out["dG"] = dA, dG
    return out, flags


def step_bn(layer, state: dict, inputs: dict, hp: dict):
    """One step of a batch-norm layer's affine parameters, the diagonal way
    [KFAC sections 1 and 5.4, R17] in both methods: the Fisher diagonal of
    gamma (weight, [C, 1]) and beta (bias, [C]) from bn_fisher, its EMA, the
    division by (F + damping_bn) (section 4.2: the batch-norm damping) and
    the momentum update; no rescaling.  Returns (new_state, flags) with
    dA = the gamma diagonal and dG = the beta diagonal."""
    f_gamma, f_beta = bn_fisher(inputs["a"], inputs["g"])
    target = np.stack([f_gamma, f_beta], axis=1)[:, :2 if layer.has_bias else 1]
    out, flags = _diagonal_tail(layer, state, inputs, hp, target, hp["damping_bn"])
    out["dA"], out["dG"] = f_gamma, f_beta
    return out, flags
