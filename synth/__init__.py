"""Seeded synthetic workloads for the K-FAC optimizer step.

This module only describes layer stacks (shapes, hyperparameters) and draws
tensors from a counter-keyed NumPy generator.  It holds none of the
optimizer's arithmetic: no factor, inverse, preconditioner or update is
computed here.  Both the float64 oracle (through the tests) and the HIP path
(through the tests and the benchmark) consume exactly the bits drawn here.

Workload shapes follow the networks the pages measure on:
  * CAFIN briefing (aiunzipped.com), "Empirical Highlights": ResNet-18 on
    image classification; the diagonal AdaFisher-style step.
  * Osawa et al., arXiv 1811.12019 (paperlayer.ai summary), section 5.1:
    ResNet-50 on ImageNet, 32 images per GPU; the full K-FAC step.
  * Transformer MLP-shaped linear stacks in bf16 (no page measures these; the
    shapes are the ones the workload description fixes).

Every tensor of a (config, step, layer, tensor) tuple is drawn in chunks of
CHUNK elements; chunk c comes from
``Generator(PCG64(SeedSequence([seed, cfg_id, step, layer, tensor, c])))``,
so any chunk can be regenerated on its own and the result does not depend on
how many threads fill the array.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

CHUNK = 1 << 22

# tensor ids inside the seed key
T_ACT, T_GRAD_OUT, T_GRAD_W, T_GRAD_B, T_W, T_B = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Layer:
    """One layer of a stack.

    Linear: activations a [rows, d_in], output gradients g [rows, d_out].
    Conv2d: input x [batch, c_in, h, w] (NCHW), output gradient
    g [batch, d_out, h_out, w_out]; d_in = c_in * k * k in (c, kh, kw) order;
    rows = batch * h_out * w_out.
    Batch norm ("bn"): normalised input x_hat and output gradient, both
    [batch, C, h, w]; d_in = 1 (gamma), d_out = C, rows = batch.
    """
    name: str
    kind: str              # "linear" | "conv" | "bn"
    d_in: int              # unfolded input width (without the bias column)
    d_out: int
    has_bias: bool
    rows: int
    batch: int = 0
    c_in: int = 0
    h: int = 0
    w: int = 0
    k: int = 1
    stride: int = 1
    pad: int = 0

    @property
    def d_a(self) -> int:
        return self.d_in + (1 if self.has_bias else 0)

    @property
    def spatial(self) -> bool:
        return self.kind in ("conv", "bn")

    @property
    def h_out(self) -> int:
        return (self.h + 2 * self.pad - self.k) // self.stride + 1 if self.spatial else 0

    @property
    def w_out(self) -> int:
        return (self.w + 2 * self.pad - self.k) // self.stride + 1 if self.spatial else 0

    @property
    def act_shape(self):
        if self.spatial:
            return (self.batch, self.c_in, self.h, self.w)
        return (self.rows, self.d_in)

    @property
    def grad_out_shape(self):
        if self.spatial:
            return (self.batch, self.d_out, self.h_out, self.w_out)
        return (self.rows, self.d_out)

    @property
    def n_params(self) -> int:
        return self.d_out * self.d_a


def conv(name, c_in, c_out, k, stride, pad, batch, h, w=None, bias=False) -> Layer:
    w = h if w is None else w
    ho = (h + 2 * pad - k) // stride + 1
    wo = (w + 2 * pad - k) // stride + 1
    return Layer(name, "conv", c_in * k * k, c_out, bias, batch * ho * wo,
                 batch, c_in, h, w, k, stride, pad)


def linear(name, d_in, d_out, rows, bias=True) -> Layer:
    return Layer(name, "linear", d_in, d_out, bias, rows)


def batchnorm(name, channels, batch, h, w=None, bias=True) -> Layer:
    """Affine parameters of a batch-norm layer over `channels` planes of h x w."""
    w = h if w is None else w
    return Layer(name, "bn", 1, channels, bias, batch, batch, channels, h, w, 1, 1, 0)


def with_batchnorm(layers) -> List[Layer]:
    """A conv stack with a batch-norm layer after every convolution (on its
    output planes), as in the ResNet families."""
    out = []
    for L in layers:
        out.append(L)
        if L.kind == "conv":
            out.append(batchnorm(L.name + ".bn", L.d_out, L.batch, L.h_out, L.w_out))
    return out


def resnet18_layers(batch=128, res=224, classes=1000) -> List[Layer]:
    """ResNet-18 (torchvision layout): 7x7/2 stem, 3x3/2 max-pool, four stages of
    two basic blocks (64/128/256/512), 1x1/2 projection on stage entry, FC with
    bias.  20 convolutions + 1 FC; 11,679,912 weights at 1000 classes."""
    L = [conv("conv1", 3, 64, 7, 2, 3, batch, res)]
    s = ((res + 6 - 7) // 2 + 1 + 2 - 3) // 2 + 1       # after stem + max-pool
    for i in range(2):
        L.append(conv(f"layer1.{i}.conv1", 64, 64, 3, 1, 1, batch, s))
        L.append(conv(f"layer1.{i}.conv2", 64, 64, 3, 1, 1, batch, s))
    cin = 64
    for li, width in ((2, 128), (3, 256), (4, 512)):
        so = (s + 2 - 3) // 2 + 1
        L.append(conv(f"layer{li}.0.conv1", cin, width, 3, 2, 1, batch, s))
        L.append(conv(f"layer{li}.0.conv2", width, width, 3, 1, 1, batch, so))
        L.append(conv(f"layer{li}.0.downsample", cin, width, 1, 2, 0, batch, s))
        L.append(conv(f"layer{li}.1.conv1", width, width, 3, 1, 1, batch, so))
        L.append(conv(f"layer{li}.1.conv2", width, width, 3, 1, 1, batch, so))
        cin, s = width, so
    L.append(linear("fc", 512, classes, batch, bias=True))
    return L


def resnet50_layers(batch=32, res=224, classes=1000) -> List[Layer]:
    """ResNet-50 v1.5 (torchvision layout: stride on the 3x3 of each stage's first
    bottleneck).  53 convolutions + FC 2048->1000 with bias; 25,503,912 weights."""
    L = [conv("conv1", 3, 64, 7, 2, 3, batch, res)]
    s = ((res + 6 - 7) // 2 + 1 + 2 - 3) // 2 + 1
    cin = 64
    for li, (width, blocks, stride) in enumerate(((64, 3, 1), (128, 4, 2), (256, 6, 2), (512, 3, 2)), 1):
        out = width * 4
        for bi in range(blocks):
            st = stride if bi == 0 else 1
            so = (s + 2 - 3) // st + 1
            L.append(conv(f"layer{li}.{bi}.conv1", cin, width, 1, 1, 0, batch, s))
            L.append(conv(f"layer{li}.{bi}.conv2", width, width, 3, st, 1, batch, s))
            L.append(conv(f"layer{li}.{bi}.conv3", width, out, 1, 1, 0, batch, so))
            if bi == 0:
                L.append(conv(f"layer{li}.{bi}.downsample", cin, out, 1, st, 0, batch, s))
            cin, s = out, so
    L.append(linear("fc", 2048, classes, batch, bias=True))
    return L


def mlp_layers(n_blocks, d_model, d_ff, tokens) -> List[Layer]:
    L = []
    for i in range(n_blocks):
        L.append(linear(f"block{i}.up", d_model, d_ff, tokens, bias=True))
        L.append(linear(f"block{i}.down", d_ff, d_model, tokens, bias=True))
    return L


@dataclasses.dataclass(frozen=True)
class Config:
    """A workload: a layer stack plus the per-step scalars and input recipe."""
    cfg_id: int
    name: str
    variant: str                     # "full" | "diag"
    layers: tuple
    steps: int
    lr: float
    momentum: float
    weight_decay: float
    ema_decay: float                 # factor EMA (full) or diagonal-FIM EMA (diag)
    damping: float
    refresh_every: int = 1           # full variant: invert when (t-1) % k == 0
    act_dtype: str = "f32"           # "f32" | "bf16"
    grad_dtype: str = "f32"
    act_std: float = 1.0
    grad_std: float = 1e-3
    relu: bool = False
    w_std: float = 0.02
    grad_w_std: float = 1e-3
    seed: int = 0
    bn_damping_scale: float = 1.0    # damping of batch-norm layers = this x damping
    rescale: bool = False            # weight rescaling after the update

    @property
    def n_params(self) -> int:
        return sum(l.n_params for l in self.layers)


def _c1(layers=None):
    return Config(0, "fc64", "full", tuple(layers or [linear("fc", 64, 32, 128, bias=True)]),
                  steps=10, lr=0.1, momentum=0.9, weight_decay=5e-4, ema_decay=0.95,
                  damping=1e-3, refresh_every=1, act_std=1.0, grad_std=1e-2, relu=False)


def _c2(layers=None):
    return Config(1, "resnet18_diag", "diag", tuple(layers or resnet18_layers()),
                  steps=100, lr=1e-3, momentum=0.9, weight_decay=5e-4, ema_decay=0.92,
                  damping=1e-3, act_std=1.0, grad_std=1e-3, relu=True)


def _c3(layers=None):
    return Config(2, "resnet50_kfac", "full", tuple(layers or resnet50_layers()),
                  steps=10, lr=0.1, momentum=0.9, weight_decay=5e-4, ema_decay=0.95,
                  damping=2.5e-4, refresh_every=1, act_std=1.0, grad_std=1e-3, relu=True)


def _c4(layers=None):
    return Config(3, "mlp24_bf16", "full", tuple(layers or mlp_layers(24, 1024, 4096, 8192)),
                  steps=100, lr=0.1, momentum=0.9, weight_decay=5e-4, ema_decay=0.95,
                  damping=1e-3, refresh_every=10, act_dtype="bf16", grad_dtype="bf16",
                  act_std=1.0, grad_std=1e-3, relu=False)


def _c5(layers=None):
    return Config(4, "pair16k_bf16", "full", tuple(layers or mlp_layers(1, 4096, 16384, 16384)),
                  steps=100, lr=0.1, momentum=0.9, weight_decay=5e-4, ema_decay=0.95,
                  damping=1e-3, refresh_every=20, act_dtype="bf16", grad_dtype="bf16",
                  act_std=1.0, grad_std=1e-3, relu=False)


def _bn50(layers=None):
    """The 53 batch-norm layers of ResNet-50 at 32 x 224^2 (one after every
    convolution, on its output planes), alone: their diagonal-Fisher step."""
    bn = [L for L in with_batchnorm(resnet50_layers()) if L.kind == "bn"]
    return Config(5, "resnet50_bn_diag", "diag", tuple(layers or bn),
                  steps=10, lr=0.1, momentum=0.9, weight_decay=5e-4, ema_decay=0.95,
                  damping=2.5e-4, act_std=1.0, grad_std=1e-3, relu=False)


def full_config(name: str) -> Config:
    """The five workloads at their stated sizes, and the batch-norm layers of
    ResNet-50 on their own."""
    return {"fc64": _c1, "resnet18_diag": _c2, "resnet50_kfac": _c3,
            "mlp24_bf16": _c4, "pair16k_bf16": _c5, "resnet50_bn_diag": _bn50}[name]()


CONFIG_NAMES = ("fc64", "resnet18_diag", "resnet50_kfac", "mlp24_bf16", "pair16k_bf16", "resnet50_bn_diag")


def small_config(name: str) -> Config:
    """Scaled-down stand-ins with the same layer kinds, kernel shapes, strides,
    bias columns and dtypes, sized so the float64 oracle finishes in seconds
    while every dimension still spans several 64/128-wide tiles plus a ragged
    tail."""
    if name == "fc64":
        return _c1()
    if name == "resnet18_diag":
        return dataclasses.replace(_c2(resnet18_layers(batch=4, res=64, classes=1000)), steps=3)
    if name == "resnet50_kfac":
        L = [conv("conv1", 3, 64, 7, 2, 3, 2, 37),
             conv("l1.conv2", 64, 64, 3, 1, 1, 2, 19),
             conv("l2.conv2", 128, 128, 3, 2, 1, 2, 19),
             conv("l2.down", 96, 300, 1, 2, 0, 2, 19),
             conv("l3.conv1", 200, 130, 1, 1, 0, 2, 10),
             conv("l4.conv2", 60, 257, 3, 1, 1, 3, 7),
             linear("fc", 300, 133, 32, bias=True)]
        return dataclasses.replace(_c3(L), steps=3)
    if name == "mlp24_bf16":
        return dataclasses.replace(_c4(mlp_layers(2, 200, 513, 700)), steps=3, refresh_every=2)
    if name == "pair16k_bf16":
        return dataclasses.replace(_c5(mlp_layers(1, 256, 1023, 900)), steps=3, refresh_every=2)
    if name == "resnet50_bn_diag":
        bn = [L for L in with_batchnorm(resnet50_layers(batch=2, res=64)) if L.kind == "bn"]
        return dataclasses.replace(_bn50(bn), steps=3)
    raise KeyError(name)


# ----------------------------------------------------------------------------
# drawing

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(key, n: int, std: float, out: Optional[np.ndarray] = None) -> np.ndarray:
    """n float32 draws of N(0, std^2), chunk-keyed (see module docstring)."""
    out = np.empty(n, np.float32) if out is None else out
    nch = (n + CHUNK - 1) // CHUNK

    def fill(c):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key) + [c])))
        sl = out[c * CHUNK:(c + 1) * CHUNK]
        g.standard_normal(out=sl, dtype=np.float32)
        if std != 1.0:
            np.multiply(sl, np.float32(std), out=sl)

    if nch <= 1:
        for c in range(nch):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Input encoding only (no NaN/Inf in the draws)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _key(cfg: Config, step: int, li: int, tensor: int):
    return (cfg.seed, cfg.cfg_id, step, li, tensor)


def draw_activation(cfg: Config, step: int, li: int) -> np.ndarray:
    """Layer li's input at step t (>=1): N(0, act_std), ReLU-clipped when the
    workload says so; float32, or bf16 bit patterns (uint16)."""
    L = cfg.layers[li]
    n = int(np.prod(L.act_shape))
    x = _normal(_key(cfg, step, li, T_ACT), n, cfg.act_std)
    if cfg.relu and L.kind != "bn":     # a batch-norm input is the normalised (unclipped) activation
        np.maximum(x, np.float32(0), out=x)
    x = x.reshape(L.act_shape)
    return to_bf16_bits(x) if cfg.act_dtype == "bf16" else x


def draw_grad_out(cfg: Config, step: int, li: int) -> np.ndarray:
    """Back-propagated output gradient of layer li at step t: N(0, grad_std)."""
    L = cfg.layers[li]
    n = int(np.prod(L.grad_out_shape))
    g = _normal(_key(cfg, step, li, T_GRAD_OUT), n, cfg.grad_std).reshape(L.grad_out_shape)
    return to_bf16_bits(g) if cfg.grad_dtype == "bf16" else g


def draw_grad_w(cfg: Config, step: int, li: int):
    """The weight gradient handed to the optimizer: N(0, grad_w_std), float32,
    [d_out, d_in] (conv: [c_out, c_in*k*k]) plus [d_out] for the bias."""
    L = cfg.layers[li]
    gw = _normal(_key(cfg, step, li, T_GRAD_W), L.d_out * L.d_in, cfg.grad_w_std).reshape(L.d_out, L.d_in)
    gb = _normal(_key(cfg, step, li, T_GRAD_B), L.d_out, cfg.grad_w_std) if L.has_bias else None
    return gw, gb


def step_inputs(cfg: Config, step: int, li: int) -> Dict[str, np.ndarray]:
    gw, gb = draw_grad_w(cfg, step, li)
    return {"a": draw_activation(cfg, step, li), "g": draw_grad_out(cfg, step, li),
            "grad_w": gw, "grad_b": gb}


def initial_state(cfg: Config, li: int) -> Dict[str, np.ndarray]:
    """Step-0 state of layer li: W ~ N(0, w_std) (bias included), zero momentum;
    full variant: A0 = I, G0 = I and zero inverses; diagonal variant: F0 = 1.
    """
    L = cfg.layers[li]
    s = {"w": _normal(_key(cfg, 0, li, T_W), L.d_out * L.d_in, cfg.w_std).reshape(L.d_out, L.d_in),
         "mom_w": np.zeros((L.d_out, L.d_in), np.float32)}
    if L.has_bias:
        s["b"] = _normal(_key(cfg, 0, li, T_B), L.d_out, cfg.w_std)
        s["mom_b"] = np.zeros(L.d_out, np.float32)
    if cfg.variant == "full" and L.kind != "bn":
        s["A"] = np.eye(L.d_a, dtype=np.float32)
        s["G"] = np.eye(L.d_out, dtype=np.float32)
        s["A_inv"] = np.zeros((L.d_a, L.d_a), np.float32)
        s["G_inv"] = np.zeros((L.d_out, L.d_out), np.float32)
    else:
        s["F_w"] = np.ones((L.d_out, L.d_in), np.float32)
        if L.has_bias:
            s["F_b"] = np.ones(L.d_out, np.float32)
    return s


def refresh_at(cfg: Config, step: int) -> bool:
    """Inverse refresh schedule: step t (1-based) refreshes when (t-1) % k == 0."""
    return (step - 1) % cfg.refresh_every == 0


def hparams(cfg: Config) -> Dict[str, float]:
    return {"lr": cfg.lr, "momentum": cfg.momentum, "weight_decay": cfg.weight_decay,
            "ema_decay": cfg.ema_decay, "damping": cfg.damping, "damping_bn": cfg.damping * cfg.bn_damping_scale,
            "rescale": cfg.rescale, "rescale_eps": 1e-9}
