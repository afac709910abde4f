"""Pins of the float64 oracle against facts fixed by the mathematics.

Each ``pin_*`` returns True when the oracle (passed in as a module-like
object, so a test can plant a mistake in a copy of it) agrees with something
other than itself: brute-force loops, a closed form, an invariant, or a
library routine that computes the same well-defined quantity.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np
import torch


class Geo:
    """Minimal layer description the oracle reads."""

    def __init__(self, kind="linear", has_bias=False, k=1, stride=1, pad=0):
        self.kind, self.has_bias, self.k, self.stride, self.pad = kind, has_bias, k, stride, pad


def hadamard(n: int) -> np.ndarray:
    """Sylvester construction: H_1 = [1], H_2m = [[H, H], [H, -H]]; H^T H = n I."""
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


# ---------------------------------------------------------------------------
# unfold

def pin_unfold_direct_conv(O, seed=0) -> bool:
    """U . W_flat^T equals a convolution written as explicit loops."""
    rng = np.random.default_rng(seed)
    B, C, H, W, Co, k, s, p = 2, 3, 5, 5, 4, 3, 2, 1
    x = rng.standard_normal((B, C, H, W))
    w = rng.standard_normal((Co, C, k, k))
    Ho = (H + 2 * p - k) // s + 1
    Wo = (W + 2 * p - k) // s + 1
    ref = np.zeros((B, Co, Ho, Wo))
    for b, o, ho, wo in itertools.product(range(B), range(Co), range(Ho), range(Wo)):
        acc = 0.0
        for c, kh, kw in itertools.product(range(C), range(k), range(k)):
            hi, wi = ho * s - p + kh, wo * s - p + kw
            if 0 <= hi < H and 0 <= wi < W:
                acc += x[b, c, hi, wi] * w[o, c, kh, kw]
        ref[b, o, ho, wo] = acc
    U = O.unfold(x, k, s, p)
    got = (U @ w.reshape(Co, -1).T).reshape(B, Ho, Wo, Co).transpose(0, 3, 1, 2)
    return U.shape == (B * Ho * Wo, C * k * k) and np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_unfold_library(O, seed=1) -> bool:
    """Same columns and rows as the library im2col (torch unfold, float64 CPU)."""
    rng = np.random.default_rng(seed)
    ok = True
    for (B, C, H, W, k, s, p) in [(2, 3, 7, 6, 3, 2, 1), (1, 2, 9, 9, 7, 2, 3), (3, 4, 5, 5, 1, 2, 0),
                                  (2, 3, 6, 6, 3, 1, 1)]:
        x = rng.standard_normal((B, C, H, W))
        ref = torch.nn.functional.unfold(torch.from_numpy(x), k, padding=p, stride=s)  # [B, Ckk, L]
        ref = ref.permute(0, 2, 1).reshape(-1, C * k * k).numpy()
        got = O.unfold(x, k, s, p)
        ok &= got.shape == ref.shape and np.array_equal(got, ref)
    return bool(ok)


# ---------------------------------------------------------------------------
# factors

def pin_factor_outer_products(O, seed=2) -> bool:
    """A-hat = (1/N) sum_n a_n a_n^T by an explicit loop; symmetric, PSD, and
    trace(A-hat) = mean squared row norm."""
    rng = np.random.default_rng(seed)
    N, d = 13, 6
    a = rng.standard_normal((N, d))
    ref = np.zeros((d, d))
    for n in range(N):
        for i in range(d):
            for j in range(d):
                ref[i, j] += a[n, i] * a[n, j]
    ref /= N
    got = O.kronecker_factor(a)
    ev = np.linalg.eigvalsh(got)
    return (np.allclose(got, ref, rtol=1e-13, atol=1e-13) and np.array_equal(got, got.T)
            and ev.min() >= -1e-12 * np.abs(ev).max()
            and np.isclose(np.trace(got), (a * a).sum(axis=1).mean(), rtol=1e-13))


def pin_factor_hadamard(O) -> bool:
    """Rows taken from a Sylvester-Hadamard matrix give A-hat = I exactly; with a
    bias the appended ones column is column 0 of H, i.e. the activations are
    columns 1..d_in of H and the factor is still I (a_bar = [a | 1])."""
    N, d_in = 32, 11
    H = hadamard(N)
    geo = Geo("linear", has_bias=True)
    a = H[:, 1:1 + d_in]
    g = 0.5 * H[:, 1:6]
    abar, grows = O.layer_rows(geo, a.astype(np.float32), g.astype(np.float32))
    A = O.kronecker_factor(abar)
    G = O.kronecker_factor(grows)
    return (abar.shape == (N, d_in + 1) and np.array_equal(abar[:, -1], np.ones(N))
            and np.array_equal(A, np.eye(d_in + 1)) and np.array_equal(G, 0.25 * np.eye(5)))


def pin_bias_column(O, seed=3) -> bool:
    """Last row/column of A-hat with a bias: the column means of a, and 1."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((20, 4)).astype(np.float32)
    g = rng.standard_normal((20, 3)).astype(np.float32)
    abar, _ = O.layer_rows(Geo("linear", has_bias=True), a, g)
    A = O.kronecker_factor(abar)
    m = a.astype(np.float64).mean(axis=0)
    return np.allclose(A[-1, :-1], m, rtol=1e-13, atol=1e-15) and np.allclose(A[:-1, -1], m) and A[-1, -1] == 1.0


def pin_conv_rows(O, seed=4) -> bool:
    """Convolution G rows: one row per (sample, output position), channel as
    column, in the same order as the unfold rows: checked by the gradient
    identity grad_W = g_rows^T U / N against an explicit loop over the
    convolution's input/output positions."""
    rng = np.random.default_rng(seed)
    B, C, H, W, Co, k, s, p = 2, 2, 5, 4, 3, 3, 2, 1
    x = rng.standard_normal((B, C, H, W)).astype(np.float32)
    Ho, Wo = (H + 2 * p - k) // s + 1, (W + 2 * p - k) // s + 1
    g = rng.standard_normal((B, Co, Ho, Wo)).astype(np.float32)
    U, grows = O.layer_rows(Geo("conv", False, k, s, p), x, g)
    gw = grows.T @ U
    ref = np.zeros((Co, C, k, k))
    for b, o, ho, wo, c, kh, kw in itertools.product(range(B), range(Co), range(Ho), range(Wo), range(C),
                                                     range(k), range(k)):
        hi, wi = ho * s - p + kh, wo * s - p + kw
        if 0 <= hi < H and 0 <= wi < W:
            ref[o, c, kh, kw] += float(g[b, o, ho, wo]) * float(x[b, c, hi, wi])
    return grows.shape == (B * Ho * Wo, Co) and np.allclose(gw, ref.reshape(Co, -1), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# single columns (the full-size checks build single factor entries from them)

# (B, C, H, W, k, stride, pad): kernel sizes 1, 2, 3 and 7, strides 1-3, and
# paddings up to 3, beyond half the kernel (taps that lie wholly in the padding
# for the first and last output rows)
COLUMN_GEOMS = [(2, 3, 5, 6, 1, 2, 1), (2, 2, 5, 5, 2, 1, 3), (1, 2, 7, 6, 3, 3, 2), (2, 2, 6, 5, 3, 1, 0),
                (1, 2, 9, 8, 7, 2, 3), (2, 1, 4, 4, 7, 1, 3), (1, 3, 8, 7, 3, 2, 3)]


def pin_unfold_column_library(O, seed=14) -> bool:
    """Every column of unfold_column equals that column of the library im2col
    (torch unfold, float64 CPU) and of the conv loops' input index
    x[b, c, ho s - p + kh, wo s - p + kw] (zero outside the image), bit for bit,
    for fp32 inputs."""
    rng = np.random.default_rng(seed)
    ok = True
    for (B, C, H, W, k, s, p) in COLUMN_GEOMS:
        x = rng.standard_normal((B, C, H, W)).astype(np.float32)
        ref = torch.nn.functional.unfold(torch.from_numpy(x.astype(np.float64)), k, padding=p, stride=s)
        ref = ref.permute(0, 2, 1).reshape(-1, C * k * k).numpy()
        Ho, Wo = (H + 2 * p - k) // s + 1, (W + 2 * p - k) // s + 1
        for j in range(C * k * k):
            col = O.unfold_column(x, k, s, p, j)
            ok &= col.dtype == np.float64 and col.shape == (B * Ho * Wo,) and np.array_equal(col, ref[:, j])
        # one column by the index formula, written as loops
        j = rng.integers(0, C * k * k)
        c, kh, kw = j // (k * k), (j // k) % k, j % k
        loop = np.zeros(B * Ho * Wo)
        for b, ho, wo in itertools.product(range(B), range(Ho), range(Wo)):
            hi, wi = ho * s - p + kh, wo * s - p + kw
            if 0 <= hi < H and 0 <= wi < W:
                loop[(b * Ho + ho) * Wo + wo] = x[b, c, hi, wi]
        ok &= np.array_equal(O.unfold_column(x, k, s, p, j), loop)
    return bool(ok)


def pin_layer_columns(O, seed=15) -> bool:
    """activation_column / gradient_column give exactly the columns of the rows
    the factors are built from: the conv input's unfold (torch im2col) with the
    constant-1 bias column last, and the output gradient with one row per
    (sample, output position) by explicit loops; linear layers' columns of a
    and g (fp32 and bf16 bit patterns) and the bias column of ones."""
    rng = np.random.default_rng(seed)
    ok = True
    for (B, C, H, W, k, s, p), bias in zip(COLUMN_GEOMS, (True, False, True, True, False, True, False)):
        geo = Geo("conv", bias, k, s, p)
        Ho, Wo = (H + 2 * p - k) // s + 1, (W + 2 * p - k) // s + 1
        Co = 3
        x = rng.standard_normal((B, C, H, W)).astype(np.float32)
        g = rng.standard_normal((B, Co, Ho, Wo)).astype(np.float32)
        U = torch.nn.functional.unfold(torch.from_numpy(x.astype(np.float64)), k, padding=p, stride=s)
        U = U.permute(0, 2, 1).reshape(-1, C * k * k).numpy()
        d_in = C * k * k
        for j in range(d_in + int(bias)):
            ref = U[:, j] if j < d_in else np.ones(B * Ho * Wo)
            ok &= np.array_equal(O.activation_column(_ColGeo(geo, d_in), x, j), ref)
        for o in range(Co):
            ref = np.zeros(B * Ho * Wo)
            for b, ho, wo in itertools.product(range(B), range(Ho), range(Wo)):
                ref[(b * Ho + ho) * Wo + wo] = g[b, o, ho, wo]
            ok &= np.array_equal(O.gradient_column(geo, g, o), ref)
    for bias, bf16 in ((True, False), (False, False), (True, True)):
        N, d_in, d_out = 9, 5, 4
        a = rng.standard_normal((N, d_in)).astype(np.float32)
        g = rng.standard_normal((N, d_out)).astype(np.float32)
        if bf16:   # truncated bf16 patterns: their float32 value is the pattern shifted up 16 bits
            a = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
            g = (g.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
            af = (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
            gf = (g.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        else:
            af, gf = a.astype(np.float64), g.astype(np.float64)
        geo = _ColGeo(Geo("linear", bias), d_in)
        for j in range(d_in + int(bias)):
            ref = af[:, j] if j < d_in else np.ones(N)
            ok &= np.array_equal(O.activation_column(geo, a, j), ref)
        for o in range(d_out):
            ok &= np.array_equal(O.gradient_column(geo, g, o), gf[:, o])
    return bool(ok)


class _ColGeo(Geo):
    """Geo plus the unfolded input width (the column helpers need d_in)."""

    def __init__(self, geo, d_in):
        super().__init__(geo.kind, geo.has_bias, geo.k, geo.stride, geo.pad)
        self.d_in = d_in


def pin_bf16_widen(O) -> bool:
    """bf16 patterns widen to the float32 whose upper half they are."""
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x3E00, 0x7F7F], np.uint16)
    ref = np.array([1.0, -1.0, 3.140625, 0.0, -0.0, 0.125, 3.3895313892515355e38])
    got = O.widen(bits)
    return got.dtype == np.float64 and np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# EMA

def pin_ema_closed_form(O) -> bool:
    """Constant input X: A_t = eps^t A_0 + (1 - eps^t) X; eps = 0 gives X,
    eps = 1 keeps A_0."""
    rng = np.random.default_rng(5)
    A0 = np.eye(4)
    X = rng.standard_normal((4, 4))
    X = X @ X.T
    ok = True
    for eps in (0.95, 0.5, 0.0, 1.0):
        A = A0
        for t in range(1, 8):
            A = O.ema(A, X, eps)
            ok &= np.allclose(A, eps ** t * A0 + (1 - eps ** t) * X, rtol=1e-12, atol=1e-14)
    return bool(ok)


# ---------------------------------------------------------------------------
# damped inverse

def pin_inverse_sherman_morrison(O) -> bool:
    """N = 1: (a a^T + lam I)^-1 = (1/lam)(I - a a^T / (lam + |a|^2))."""
    rng = np.random.default_rng(6)
    ok = True
    for d, lam in ((5, 1e-3), (9, 0.5), (1, 2.0)):
        a = rng.standard_normal(d)
        ref = (np.eye(d) - np.outer(a, a) / (lam + a @ a)) / lam
        got = O.damped_inverse(O.kronecker_factor(a[None, :]), lam)
        ok &= np.allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    return bool(ok)


def pin_inverse_diagonal_and_residual(O) -> bool:
    """Diagonal F: 1/(f_ii + lam); general SPD: (F + lam I) X = I and X equals
    the library's general inverse."""
    rng = np.random.default_rng(7)
    f = rng.uniform(0.0, 3.0, 7)
    ok = np.allclose(O.damped_inverse(np.diag(f), 0.25), np.diag(1.0 / (f + 0.25)), rtol=1e-14)
    a = rng.standard_normal((40, 12))
    F = a.T @ a / 40
    X = O.damped_inverse(F, 1e-3)
    M = F + 1e-3 * np.eye(12)
    ok &= np.allclose(M @ X, np.eye(12), atol=1e-10)
    ok &= np.allclose(X, np.linalg.inv(M), rtol=1e-9, atol=1e-9 * np.abs(X).max())
    ok &= np.array_equal(X, X.T)
    return bool(ok)


def pin_inverse_not_pd_raises(O) -> bool:
    F = np.diag([1.0, -1.0, 2.0])
    try:
        O.damped_inverse(F, 0.5)
    except np.linalg.LinAlgError:
        return True
    return False


# ---------------------------------------------------------------------------
# preconditioning

def pin_kronecker_identity(O, seed=8) -> bool:
    """((G + lam I) kron (A + lam I))^-1 vec_r(grad) = vec_r(G_inv grad A_inv),
    with the explicit Kronecker product and a dense solve (row-major vec)."""
    rng = np.random.default_rng(seed)
    ok = True
    for dg, da, lam in ((3, 5, 1e-2), (6, 7, 0.3), (4, 4, 1e-3), (1, 6, 1.0)):
        a = rng.standard_normal((11, da))
        g = rng.standard_normal((9, dg))
        A = O.kronecker_factor(a)
        G = O.kronecker_factor(g)
        grad = rng.standard_normal((dg, da))
        big = np.kron(G + lam * np.eye(dg), A + lam * np.eye(da))
        ref = np.linalg.solve(big, grad.reshape(-1)).reshape(dg, da)
        got = O.precondition(O.damped_inverse(G, lam), grad, O.damped_inverse(A, lam))
        ok &= np.allclose(got, ref, rtol=1e-8, atol=1e-8 * np.abs(ref).max())
    return bool(ok)


def pin_full_step_hadamard(O) -> bool:
    """Hadamard rows with eps = 0: A-hat = I, G-hat = c I, so the first step's
    direction is grad / ((1 + lam)(c + lam)), and with V0 = 0 the update is
    W1 = W0 - lr (P + wd W0)."""
    N, d_in, d_out, c, lam = 64, 9, 5, 0.25, 0.1
    H = hadamard(N)
    geo = Geo("linear", has_bias=True)
    rng = np.random.default_rng(9)
    st = {"w": rng.standard_normal((d_out, d_in)), "b": rng.standard_normal(d_out),
          "mom_w": np.zeros((d_out, d_in)), "mom_b": np.zeros(d_out),
          "A": np.eye(d_in + 1), "G": np.eye(d_out), "A_inv": np.zeros((d_in + 1,) * 2),
          "G_inv": np.zeros((d_out,) * 2)}
    inp = {"a": H[:, 1:1 + d_in], "g": np.sqrt(c) * H[:, 1:1 + d_out],
           "grad_w": rng.standard_normal((d_out, d_in)), "grad_b": rng.standard_normal(d_out)}
    hp = {"lr": 0.1, "momentum": 0.9, "weight_decay": 5e-4, "ema_decay": 0.0, "damping": lam}
    out, flags = O.step_full(geo, st, inp, hp, refresh=True)
    gaug = np.concatenate([inp["grad_w"], inp["grad_b"][:, None]], 1)
    waug = np.concatenate([st["w"], st["b"][:, None]], 1)
    P = gaug / ((1 + lam) * (c + lam))
    W1 = waug - 0.1 * (P + 5e-4 * waug)
    got = np.concatenate([out["w"], out["b"][:, None]], 1)
    return flags == 0 and np.allclose(out["P"], P, rtol=1e-12) and np.allclose(got, W1, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# update

def _sgd_loop(w0, grads, lr, mu, wd):
    """Plain SGD with heavy-ball momentum and L2 weight decay, element by element."""
    w = [list(r) for r in w0]
    v = [[0.0] * len(r) for r in w0]
    for gr in grads:
        for i in range(len(w)):
            for j in range(len(w[i])):
                d = gr[i][j] + wd * w[i][j]
                v[i][j] = mu * v[i][j] + d
                w[i][j] = w[i][j] - lr * v[i][j]
    return np.array(w)


def pin_sgd_reduction(O, seed=10) -> bool:
    """eps = 0 with identity inverses kept (no refresh): the full step is SGD
    with momentum and weight decay -- equal to an element-wise loop and to
    torch.optim.SGD (float64, CPU) over several steps."""
    rng = np.random.default_rng(seed)
    d_out, d_in, T = 3, 4, 5
    geo = Geo("linear", has_bias=True)
    w0 = rng.standard_normal((d_out, d_in))
    b0 = rng.standard_normal(d_out)
    st = {"w": w0, "b": b0, "mom_w": np.zeros_like(w0), "mom_b": np.zeros_like(b0),
          "A": np.eye(d_in + 1), "G": np.eye(d_out), "A_inv": np.eye(d_in + 1), "G_inv": np.eye(d_out)}
    hp = {"lr": 0.1, "momentum": 0.9, "weight_decay": 5e-4, "ema_decay": 0.0, "damping": 1e-3}
    grads = []
    p = torch.tensor(np.concatenate([w0, b0[:, None]], 1), requires_grad=True)
    opt = torch.optim.SGD([p], lr=0.1, momentum=0.9, weight_decay=5e-4)
    for t in range(T):
        inp = {"a": rng.standard_normal((7, d_in)), "g": rng.standard_normal((7, d_out)),
               "grad_w": rng.standard_normal((d_out, d_in)), "grad_b": rng.standard_normal(d_out)}
        gaug = np.concatenate([inp["grad_w"], inp["grad_b"][:, None]], 1)
        grads.append(gaug.tolist())
        out, _ = O.step_full(geo, st, inp, hp, refresh=False)
        st = dict(st, **{k: out[k] for k in ("w", "b", "mom_w", "mom_b", "A", "G")})
        p.grad = torch.tensor(gaug)
        opt.step()
    got = np.concatenate([st["w"], st["b"][:, None]], 1)
    ref = _sgd_loop(np.concatenate([w0, b0[:, None]], 1).tolist(), grads, 0.1, 0.9, 5e-4)
    return np.allclose(got, ref, rtol=1e-13, atol=1e-15) and np.allclose(got, p.detach().numpy(), rtol=1e-13)


def pin_momentum_constant_direction(O) -> bool:
    """Constant D and wd = 0: V_t = D (1 - mu^t) / (1 - mu)."""
    D = np.array([[1.0, -2.0], [0.5, 3.0]])
    w, v = np.zeros((2, 2)), np.zeros((2, 2))
    ok = True
    for t in range(1, 10):
        w, v = O.momentum_update(w, v, D, 0.1, 0.9, 0.0)
        ok &= np.allclose(v, D * (1 - 0.9 ** t) / (1 - 0.9), rtol=1e-13)
    return bool(ok)


# ---------------------------------------------------------------------------
# diagonal variant

def pin_diag_is_factor_diagonal(O, seed=11) -> bool:
    """dA = diag(A-hat), dG = diag(G-hat) for linear and conv layers; the
    per-parameter product dG[o] dA[j] is the diagonal of G-hat kron A-hat in
    row-major [d_out, d_a] order."""
    rng = np.random.default_rng(seed)
    ok = True
    cases = [(Geo("linear", True), rng.standard_normal((15, 6)), rng.standard_normal((15, 4))),
             (Geo("conv", False, 3, 2, 1), rng.standard_normal((2, 3, 7, 6)), rng.standard_normal((2, 4, 4, 3))),
             (Geo("conv", True, 1, 1, 0), rng.standard_normal((2, 3, 4, 4)), rng.standard_normal((2, 5, 4, 4)))]
    for geo, a, g in cases:
        dA, dG = O.diag_factors(geo, a, g)
        abar, grows = O.layer_rows(geo, a, g)
        A, G = O.kronecker_factor(abar), O.kronecker_factor(grows)
        ok &= np.allclose(dA, np.diag(A), rtol=1e-13) and np.allclose(dG, np.diag(G), rtol=1e-13)
        ok &= np.allclose(np.diag(np.kron(G, A)).reshape(len(dG), len(dA)), np.outer(dG, dA), rtol=1e-13)
    return bool(ok)


def pin_diag_conv_window_sums(O, seed=12) -> bool:
    """Conv dA[c, kh, kw] = (1/N) sum over samples and output positions of
    x[b, c, ho*s - p + kh, wo*s - p + kw]^2 (zero outside), by loops."""
    rng = np.random.default_rng(seed)
    B, C, H, W, Co, k, s, p = 2, 2, 7, 5, 3, 3, 2, 1
    x = rng.standard_normal((B, C, H, W))
    Ho, Wo = (H + 2 * p - k) // s + 1, (W + 2 * p - k) // s + 1
    g = rng.standard_normal((B, Co, Ho, Wo))
    dA, dG = O.diag_factors(Geo("conv", False, k, s, p), x, g)
    N = B * Ho * Wo
    ref = np.zeros((C, k, k))
    for b, c, kh, kw, ho, wo in itertools.product(range(B), range(C), range(k), range(k), range(Ho), range(Wo)):
        hi, wi = ho * s - p + kh, wo * s - p + kw
        if 0 <= hi < H and 0 <= wi < W:
            ref[c, kh, kw] += x[b, c, hi, wi] ** 2
    refG = np.array([(g[:, o] ** 2).sum() for o in range(Co)]) / N
    return np.allclose(dA, ref.reshape(-1) / N, rtol=1e-13) and np.allclose(dG, refG, rtol=1e-13)


def pin_diag_step_closed_form(O, seed=13) -> bool:
    """beta = 0: F = dG dA^T, P = grad / (F + lam) element by element; beta = 1
    with F0 = 1 - lam: P = grad, and steps reduce to the SGD loop."""
    rng = np.random.default_rng(seed)
    geo = Geo("linear", True)
    d_in, d_out, N = 5, 3, 8
    a = rng.standard_normal((N, d_in))
    g = rng.standard_normal((N, d_out))
    w0, b0 = rng.standard_normal((d_out, d_in)), rng.standard_normal(d_out)
    gw, gb = rng.standard_normal((d_out, d_in)), rng.standard_normal(d_out)
    st = {"w": w0, "b": b0, "mom_w": np.zeros_like(w0), "mom_b": np.zeros_like(b0),
          "F_w": np.full_like(w0, 7.0), "F_b": np.full_like(b0, 7.0)}
    inp = {"a": a, "g": g, "grad_w": gw, "grad_b": gb}
    lam = 1e-2
    out, _ = O.step_diag(geo, st, inp, {"lr": 0.1, "momentum": 0.9, "weight_decay": 0.0,
                                        "ema_decay": 0.0, "damping": lam})
    ok = True
    for o in range(d_out):
        for j in range(d_in + 1):
            dAj = np.mean(a[:, j] ** 2) if j < d_in else 1.0
            dGo = np.mean(g[:, o] ** 2)
            gr = gw[o, j] if j < d_in else gb[o]
            ok &= np.isclose(out["P"][o, j], gr / (dGo * dAj + lam), rtol=1e-12)
    # SGD reduction
    st = dict(st, F_w=np.full_like(w0, 1 - lam), F_b=np.full_like(b0, 1 - lam))
    hp = {"lr": 0.05, "momentum": 0.9, "weight_decay": 5e-4, "ema_decay": 1.0, "damping": lam}
    grads = []
    for t in range(4):
        gw, gb = rng.standard_normal((d_out, d_in)), rng.standard_normal(d_out)
        grads.append(np.concatenate([gw, gb[:, None]], 1).tolist())
        out, _ = O.step_diag(geo, st, {"a": a, "g": g, "grad_w": gw, "grad_b": gb}, hp)
        st = dict(st, **{k: out[k] for k in ("w", "b", "mom_w", "mom_b", "F_w", "F_b")})
    ref = _sgd_loop(np.concatenate([w0, b0[:, None]], 1).tolist(), grads, 0.05, 0.9, 5e-4)
    ok &= np.allclose(np.concatenate([st["w"], st["b"][:, None]], 1), ref, rtol=1e-12, atol=1e-15)
    return bool(ok)


def pin_refresh_keeps_inverses(O) -> bool:
    """Without a refresh the previous inverses are used unchanged; a factor that
    is not positive definite keeps its inverse and raises the NOT_PD flag."""
    rng = np.random.default_rng(14)
    geo = Geo("linear", False)
    st = {"w": rng.standard_normal((2, 3)), "mom_w": np.zeros((2, 3)),
          "A": np.diag([1.0, -5.0, 1.0]), "G": np.eye(2),
          "A_inv": 2 * np.eye(3), "G_inv": 3 * np.eye(2)}
    inp = {"a": np.zeros((4, 3)), "g": np.zeros((4, 2)), "grad_w": np.ones((2, 3))}
    hp = {"lr": 0.1, "momentum": 0.0, "weight_decay": 0.0, "ema_decay": 1.0, "damping": 0.1}
    out, flags = O.step_full(geo, st, inp, hp, refresh=False)
    ok = flags == 0 and np.array_equal(out["P"], 6 * np.ones((2, 3)))
    out, flags = O.step_full(geo, st, inp, hp, refresh=True)
    ok &= flags == O.FLAG_NOT_PD and np.array_equal(out["A_inv"], 2 * np.eye(3))
    ok &= np.allclose(out["G_inv"], np.eye(2) / 1.1)
    return bool(ok)


def _gauss_jordan_inverse(M):
    """Exact inverse of a small rational matrix (Gauss-Jordan with row swaps)."""
    n = len(M)
    aug = [list(M[i]) + [Fraction(int(i == j)) for j in range(n)] for i in range(n)]
    for c in range(n):
        piv = next(r for r in range(c, n) if aug[r][c] != 0)
        aug[c], aug[piv] = aug[piv], aug[c]
        pv = aug[c][c]
        aug[c] = [x / pv for x in aug[c]]
        for r in range(n):
            if r != c and aug[r][c] != 0:
                f = aug[r][c]
                aug[r] = [x - f * y for x, y in zip(aug[r], aug[c])]
    return [row[n:] for row in aug]


def _mm(X, Y):
    return [[sum(X[i][k] * Y[k][j] for k in range(len(Y))) for j in range(len(Y[0]))] for i in range(len(X))]


def pin_full_step_exact_rational(O) -> bool:
    """Two whole steps of a tiny biased linear layer in exact rational
    arithmetic: outer-product sums, the EMA, damped inverses by Gauss-Jordan
    elimination (not Cholesky), the two-sided product, weight decay and
    momentum, in the step order the pages give.  The float64 oracle must agree
    to rounding."""
    F = Fraction
    eps, lam, lr, mu, wd = F(1, 2), F(1, 10), F(1, 4), F(9, 10), F(1, 20)
    a_steps = [[[1, 2], [3, -1], [0, 1]], [[2, 0], [-1, 1], [1, 1]]]
    g_steps = [[[1, -1], [2, 0], [0, 3]], [[1, 1], [-2, 1], [1, 0]]]
    gw_steps = [[[1, 2, -1], [0, 1, 3]], [[-1, 0, 2], [1, 1, 1]]]
    W = [[F(1), F(-2), F(1, 2)], [F(3), F(0), F(-1)]]
    V = [[F(0)] * 3 for _ in range(2)]
    A = [[F(int(i == j)) for j in range(3)] for i in range(3)]
    G = [[F(int(i == j)) for j in range(2)] for i in range(2)]
    st = {"w": np.array([[1.0, -2.0], [3.0, 0.0]]), "b": np.array([0.5, -1.0]),
          "mom_w": np.zeros((2, 2)), "mom_b": np.zeros(2), "A": np.eye(3), "G": np.eye(2),
          "A_inv": np.zeros((3, 3)), "G_inv": np.zeros((2, 2))}
    hp = {"lr": 0.25, "momentum": 0.9, "weight_decay": 0.05, "ema_decay": 0.5, "damping": 0.1}
    ok = True
    for t in range(2):
        abar = [[F(x) for x in row] + [F(1)] for row in a_steps[t]]
        g = [[F(x) for x in row] for row in g_steps[t]]
        N = len(abar)
        Ahat = [[sum(abar[n][i] * abar[n][j] for n in range(N)) / N for j in range(3)] for i in range(3)]
        Ghat = [[sum(g[n][i] * g[n][j] for n in range(N)) / N for j in range(2)] for i in range(2)]
        A = [[eps * A[i][j] + (1 - eps) * Ahat[i][j] for j in range(3)] for i in range(3)]
        G = [[eps * G[i][j] + (1 - eps) * Ghat[i][j] for j in range(2)] for i in range(2)]
        Ai = _gauss_jordan_inverse([[A[i][j] + (lam if i == j else 0) for j in range(3)] for i in range(3)])
        Gi = _gauss_jordan_inverse([[G[i][j] + (lam if i == j else 0) for j in range(2)] for i in range(2)])
        Pm = _mm(_mm(Gi, [[F(x) for x in r] for r in gw_steps[t]]), Ai)
        for i in range(2):
            for j in range(3):
                d = Pm[i][j] + wd * W[i][j]
                V[i][j] = mu * V[i][j] + d
                W[i][j] = W[i][j] - lr * V[i][j]
        gw = np.array(gw_steps[t], np.float64)
        inp = {"a": np.array(a_steps[t], np.float64), "g": np.array(g_steps[t], np.float64),
               "grad_w": gw[:, :2], "grad_b": gw[:, 2]}
        out, flags = O.step_full(Geo("linear", True), st, inp, hp, refresh=True)
        st = dict(st, **{k: out[k] for k in ("w", "b", "mom_w", "mom_b", "A", "G", "A_inv", "G_inv")})
        Wf = np.array([[float(x) for x in r] for r in W])
        got = np.concatenate([st["w"], st["b"][:, None]], 1)
        ok &= flags == 0 and np.allclose(got, Wf, rtol=1e-13, atol=1e-14)
        ok &= np.allclose(st["A_inv"], np.array([[float(x) for x in r] for r in Ai]), rtol=1e-12, atol=1e-13)
    return bool(ok)


# ---------------------------------------------------------------------------
# batch normalisation (diagonal Fisher), weight rescaling, schedule, packing

def pin_bn_fisher_autograd(O, seed=16) -> bool:
    """The batch-norm Fisher diagonal equals the mean over samples of the
    squared per-sample gradients of gamma and beta, each computed by torch
    autograd (float64, CPU) through y = gamma x_hat + beta with the sample's
    loss sum(g_b * y_b); a constant x_hat = 1, g = c gives (H W c)^2 exactly."""
    rng = np.random.default_rng(seed)
    B, C, H, W = 3, 2, 2, 3
    xhat = rng.standard_normal((B, C, H, W))
    g = rng.standard_normal((B, C, H, W))
    gamma = torch.tensor(rng.standard_normal(C), requires_grad=True)
    beta = torch.tensor(rng.standard_normal(C), requires_grad=True)
    sq_g, sq_b = np.zeros(C), np.zeros(C)
    for b in range(B):
        y = gamma[:, None, None] * torch.from_numpy(xhat[b]) + beta[:, None, None]
        dg, db = torch.autograd.grad((torch.from_numpy(g[b]) * y).sum(), (gamma, beta))
        sq_g += dg.numpy() ** 2
        sq_b += db.numpy() ** 2
    fg, fb = O.bn_fisher(xhat.astype(np.float32), g.astype(np.float32))
    fg32, fb32 = O.bn_fisher(xhat, g)
    ones = np.ones((2, 3, 4, 5))
    cg, cb = O.bn_fisher(ones, 0.5 * ones)
    return (np.allclose(fg32, sq_g / B, rtol=1e-12) and np.allclose(fb32, sq_b / B, rtol=1e-12)
            and fg.shape == (C,) and np.allclose(fg, fg32, rtol=1e-5)
            and np.array_equal(cg, np.full(3, 100.0)) and np.array_equal(cb, np.full(3, 100.0)))


def pin_bn_step_closed_form(O, seed=17) -> bool:
    """A batch-norm step at EMA decay 0: F becomes the Fisher diagonal
    (gamma in the weight column, beta in the bias column), the gradient is
    divided by F + damping_bn (not the layer damping), then the momentum
    update, element by element; dA / dG carry the two diagonals."""
    rng = np.random.default_rng(seed)
    B, C, H, W = 4, 3, 2, 2
    xhat = rng.standard_normal((B, C, H, W)).astype(np.float32)
    g = rng.standard_normal((B, C, H, W)).astype(np.float32)
    x64, g64 = xhat.astype(np.float64), g.astype(np.float64)
    fg = np.array([np.mean([np.sum(g64[b, c] * x64[b, c]) ** 2 for b in range(B)]) for c in range(C)])
    fb = np.array([np.mean([np.sum(g64[b, c]) ** 2 for b in range(B)]) for c in range(C)])
    geo = Geo("bn", True)
    st = {"w": rng.standard_normal((C, 1)), "b": rng.standard_normal(C), "mom_w": rng.standard_normal((C, 1)),
          "mom_b": rng.standard_normal(C), "F_w": np.full((C, 1), 5.0), "F_b": np.full(C, 5.0)}
    inp = {"a": xhat, "g": g, "grad_w": rng.standard_normal((C, 1)), "grad_b": rng.standard_normal(C)}
    hp = {"lr": 0.1, "momentum": 0.9, "weight_decay": 1e-2, "ema_decay": 0.0, "damping": 7.0, "damping_bn": 0.05}
    out, flags = O.step_bn(geo, st, inp, hp)
    ok = flags == 0 and np.allclose(out["dA"], fg, rtol=1e-12) and np.allclose(out["dG"], fb, rtol=1e-12)
    for c in range(C):
        for key, wk, vk, fk, f in (("grad_w", "w", "mom_w", "F_w", fg[c]), ("grad_b", "b", "mom_b", "F_b", fb[c])):
            gr = np.ravel(inp[key])[c]
            w0, v0 = np.ravel(st[wk])[c], np.ravel(st[vk])[c]
            v1 = 0.9 * v0 + gr / (f + 0.05) + 1e-2 * w0
            ok &= np.isclose(np.ravel(out[fk])[c], f, rtol=1e-12)
            ok &= np.isclose(np.ravel(out[vk])[c], v1, rtol=1e-12) and np.isclose(np.ravel(out[wk])[c], w0 - 0.1 * v1,
                                                                                  rtol=1e-12)
    return bool(ok)


def pin_rescale_norm(O, seed=18) -> bool:
    """Rescaled weights point the same way with Frobenius norm
    sqrt(2 d_out) ||W|| / (||W|| + eps) (np.linalg.norm); a He-initialised
    d_out x d_in weight (std sqrt(2 / d_in)) is left almost unchanged, which
    fixes d_out (not d_in) in the target; in a full step only the weight is
    rescaled, the bias is not."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((30, 7))
    ok = True
    for eps in (0.0, 1e-9, 0.5):
        R = O.rescale_weights(W, 30, eps)
        n = np.linalg.norm(W)
        ok &= np.isclose(np.linalg.norm(R), np.sqrt(60.0) * n / (n + eps), rtol=1e-13)
        ok &= np.isclose(np.sum(R * W) / (np.linalg.norm(R) * n), 1.0, rtol=1e-13)
    He = rng.standard_normal((400, 50)) * np.sqrt(2.0 / 50)
    ratio = np.linalg.norm(O.rescale_weights(He, 400, 1e-9)) / np.linalg.norm(He)
    ok &= abs(ratio - 1.0) < 0.02
    geo = Geo("linear", True)
    st = {"w": rng.standard_normal((3, 4)), "b": rng.standard_normal(3), "mom_w": np.zeros((3, 4)), "mom_b": np.zeros(3),
          "A": np.eye(5), "G": np.eye(3), "A_inv": np.eye(5), "G_inv": np.eye(3)}
    inp = {"a": rng.standard_normal((6, 4)), "g": rng.standard_normal((6, 3)), "grad_w": rng.standard_normal((3, 4)),
           "grad_b": rng.standard_normal(3)}
    hp = {"lr": 0.1, "momentum": 0.9, "weight_decay": 0.0, "ema_decay": 0.5, "damping": 0.1, "rescale_eps": 1e-9}
    plain, _ = O.step_full(geo, st, inp, hp, False)
    resc, _ = O.step_full(geo, st, inp, dict(hp, rescale=True), False)
    ok &= np.isclose(np.linalg.norm(resc["w"]), np.sqrt(6.0), rtol=1e-9)
    ok &= np.array_equal(resc["b"], plain["b"]) and np.allclose(resc["w"] / np.linalg.norm(resc["w"]),
                                                                  plain["w"] / np.linalg.norm(plain["w"]), rtol=1e-12)
    return bool(ok)


def pin_schedule(O) -> bool:
    """Warm-up damping: step 1 uses gamma(0), steps after t_warmup the target;
    the mid-warm-up step takes the arithmetic (linear) or geometric
    (geometric) mean; the damping never increases; batch norm scales it by
    rho_BN.  Refresh: step 1 and the dense steps refresh both; over steps
    1..T the number of A refreshes is D + floor((T - D) / k_A) (and G's with
    k_G), with refreshes exactly k apart after the dense steps."""
    ok = True
    for shape in ("linear", "geometric"):
        s = {"damping_init": 0.04, "damping_target": 0.0025, "warmup_steps": 10, "warmup_shape": shape,
             "bn_damping_scale": 16.0, "dense_steps": 7, "refresh_every_a": 5, "refresh_every_g": 3}
        lam = [O.schedule(s, t)[0] for t in range(1, 30)]
        mid = O.schedule(s, 6)[0]
        ok &= lam[0] == 0.04 and all(abs(x - 0.0025) < 1e-15 for x in lam[10:])
        ok &= all(b <= a + 1e-18 for a, b in zip(lam, lam[1:]))
        ok &= np.isclose(mid, (0.04 + 0.0025) / 2 if shape == "linear" else np.sqrt(0.04 * 0.0025), rtol=1e-12)
        ok &= np.isclose(O.schedule(s, 3)[1], 16.0 * O.schedule(s, 3)[0], rtol=1e-15)
        T = 40
        ra = [t for t in range(1, T + 1) if O.schedule(s, t)[2]]
        rg = [t for t in range(1, T + 1) if O.schedule(s, t)[3]]
        ok &= len(ra) == 7 + (T - 7) // 5 and len(rg) == 7 + (T - 7) // 3
        ok &= ra[:7] == list(range(1, 8)) and all(b - a == 5 for a, b in zip(ra[6:], ra[7:]))
        ok &= all(b - a == 3 for a, b in zip(rg[6:], rg[7:]))
    s0 = {"damping_init": 1.0, "damping_target": 0.5, "warmup_steps": 0, "warmup_shape": "linear",
          "bn_damping_scale": 1.0, "dense_steps": 0, "refresh_every_a": 4, "refresh_every_g": 4}
    ok &= O.schedule(s0, 1)[0] == 0.5 and O.schedule(s0, 1)[2] and O.schedule(s0, 1)[3]
    ok &= [t for t in range(1, 12) if O.schedule(s0, t)[2]] == [1, 5, 9]
    return bool(ok)


def pin_pack_upper(O, seed=19) -> bool:
    """Packed storage lists the upper triangle row by row: enumerating the
    pairs i <= j in row-major order gives the same sequence; d (d + 1) / 2
    entries; unpacking restores a symmetric matrix."""
    rng = np.random.default_rng(seed)
    ok = True
    for d in (1, 2, 5, 8):
        M = rng.standard_normal((d, d))
        M = M + M.T
        p = O.pack_upper(M)
        ref = [M[i, j] for i in range(d) for j in range(d) if i <= j]
        ok &= p.shape == (d * (d + 1) // 2,) and np.array_equal(p, np.array(ref))
        ok &= np.array_equal(O.unpack_upper(p, d), M)
    return bool(ok)


ALL_PINS = [pin_full_step_exact_rational, pin_unfold_direct_conv, pin_unfold_library, pin_factor_outer_products, pin_factor_hadamard,
            pin_bias_column, pin_conv_rows, pin_unfold_column_library, pin_layer_columns, pin_bf16_widen, pin_ema_closed_form,
            pin_inverse_sherman_morrison, pin_inverse_diagonal_and_residual, pin_inverse_not_pd_raises,
            pin_kronecker_identity, pin_full_step_hadamard, pin_sgd_reduction,
            pin_momentum_constant_direction, pin_diag_is_factor_diagonal, pin_diag_conv_window_sums,
            pin_diag_step_closed_form, pin_refresh_keeps_inverses, pin_bn_fisher_autograd,
            pin_bn_step_closed_form, pin_rescale_norm, pin_schedule, pin_pack_upper]
