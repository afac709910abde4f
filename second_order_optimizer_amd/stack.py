"""Device state for a stack of layers, held in torch tensors, plus the C
descriptor array pointing at it.  Allocation and marshalling only: the step
itself is one call into libkfac.so.

A layer shape is any object with the attributes ``kind`` ("linear" | "conv" |
"bn"), ``d_in``, ``d_out``, ``has_bias``, ``rows`` and, for convolutions and
batch norm, ``batch``, ``c_in``, ``h``, ``w``, ``k``, ``stride``, ``pad``,
``h_out``, ``w_out``.  With ``factor_layout="packed"`` the full method's A and
G buffers hold the packed upper triangle (d (d + 1) / 2 floats, row after row)
and are set and read in that form.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import (BATCHNORM, BF16, CONV2D, F32, FACTORS_FULL, FACTORS_PACKED, LINEAR, MODE_DIAG, MODE_FULL, OPT_RESCALE,
               REFRESH_A, REFRESH_G, HParams, hparams, layer_array, make_layer, read_flags, step_diag, step_full,
               workspace_size)

INPUT_NAMES = ("a", "g", "grad_w", "grad_b")


def _to_device(arr: np.ndarray, dev) -> torch.Tensor:
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


class KfacStack:
    """Buffers for one optimizer over `shapes` on one GPU.

    variant: "full" or "diag".  `pool` input sets are allocated so that
    successive steps can read different (pre-loaded) batches without copies.
    """

    def __init__(self, shapes: Sequence, variant: str, act_dtype: str = "f32", grad_dtype: str = "f32",
                 device="cuda", pool: int = 1, factor_layout: str = "full", inputs_from: "KfacStack" = None):
        self.shapes = list(shapes)
        self.packed = factor_layout == "packed"
        self.variant = variant
        self.mode = MODE_FULL if variant == "full" else MODE_DIAG
        self.dev = torch.device(device)
        self.adt = torch.bfloat16 if act_dtype == "bf16" else torch.float32
        self.gdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
        self.act_code = BF16 if act_dtype == "bf16" else F32
        self.grad_code = BF16 if grad_dtype == "bf16" else F32
        self.state: List[Dict[str, torch.Tensor]] = []
        self.inputs: List[List[Dict[str, Optional[torch.Tensor]]]] = []
        for L in self.shapes:
            st = self._alloc_state(L)
            self.state.append(st)
        if inputs_from is not None:       # read the input buffers of another stack of the same shapes
            self.inputs = inputs_from.inputs
        else:
            for _ in range(pool):
                self.inputs.append([self._alloc_inputs(L) for L in self.shapes])
        self.active = 0
        self._descs = {}          # one descriptor array per input slot (the buffers never move)
        self._build_desc()
        self.ws_bytes = workspace_size(self.desc, self.mode)
        self._ws = torch.zeros(self.ws_bytes + 256, dtype=torch.uint8, device=self.dev)
        base = self._ws.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256

    # -- allocation -------------------------------------------------------
    def _alloc_state(self, L) -> Dict[str, torch.Tensor]:
        f = dict(dtype=torch.float32, device=self.dev)
        d_a = L.d_in + int(L.has_bias)
        st = {"w": torch.zeros(L.d_out, L.d_in, **f), "mom_w": torch.zeros(L.d_out, L.d_in, **f)}
        if L.has_bias:
            st["b"] = torch.zeros(L.d_out, **f)
            st["mom_b"] = torch.zeros(L.d_out, **f)
        if self.variant == "full" and L.kind != "bn":
            if self.packed:
                st["A"] = torch.zeros(d_a * (d_a + 1) // 2, **f)
                st["G"] = torch.zeros(L.d_out * (L.d_out + 1) // 2, **f)
            else:
                st["A"] = torch.eye(d_a, **f)
                st["G"] = torch.eye(L.d_out, **f)
            st["A_inv"] = torch.zeros(d_a, d_a, **f)
            st["G_inv"] = torch.zeros(L.d_out, L.d_out, **f)
        else:
            st["F_w"] = torch.ones(L.d_out, L.d_in, **f)
            if L.has_bias:
                st["F_b"] = torch.ones(L.d_out, **f)
            # a batch-norm layer's dA / dG hold the gamma / beta Fisher diagonals, one entry per channel
            st["dA"] = torch.zeros(L.d_out if L.kind == "bn" else d_a, **f)
            st["dG"] = torch.zeros(L.d_out, **f)
        return st

    def _alloc_inputs(self, L) -> Dict[str, Optional[torch.Tensor]]:
        if L.kind in ("conv", "bn"):
            ashape = (L.batch, L.c_in, L.h, L.w)
            gshape = (L.batch, L.d_out, L.h_out, L.w_out)
        else:
            ashape = (L.rows, L.d_in)
            gshape = (L.rows, L.d_out)
        bn = L.kind == "bn"    # batch-norm inputs are float32
        return {"a": torch.zeros(ashape, dtype=torch.float32 if bn else self.adt, device=self.dev),
                "g": torch.zeros(gshape, dtype=torch.float32 if bn else self.gdt, device=self.dev),
                "grad_w": torch.zeros(L.d_out, L.d_in, dtype=torch.float32, device=self.dev),
                "grad_b": torch.zeros(L.d_out, dtype=torch.float32, device=self.dev) if L.has_bias else None}

    def _build_desc(self):
        if self.active in self._descs:
            self.desc = self._descs[self.active]
            return
        descs = []
        for li, L in enumerate(self.shapes):
            t = dict(self.state[li])
            t.update({k: v for k, v in self.inputs[self.active][li].items() if v is not None})
            conv = L.kind in ("conv", "bn")
            kind = {"conv": CONV2D, "bn": BATCHNORM}.get(L.kind, LINEAR)
            bn = L.kind == "bn"
            descs.append(make_layer(
                kind, L.d_in, L.d_out, L.rows, L.has_bias,
                act_dtype=F32 if bn else self.act_code, grad_dtype=F32 if bn else self.grad_code,
                batch=L.batch if conv else 0, c_in=L.c_in if conv else 0, height=L.h if conv else 0,
                width=L.w if conv else 0, k=L.k if conv else 0, stride=L.stride if conv else 0,
                pad=L.pad if conv else 0, factor_layout=FACTORS_PACKED if self.packed else FACTORS_FULL, **t))
        self.desc = layer_array(descs)
        self._descs[self.active] = self.desc

    # -- data movement ----------------------------------------------------
    def set_inputs(self, li: int, arrays: Dict[str, np.ndarray], slot: int = 0):
        for name in INPUT_NAMES:
            arr = arrays.get(name)
            if arr is None:
                continue
            dst = self.inputs[slot][li][name]
            dst.copy_(_to_device(arr, self.dev).reshape(dst.shape))

    def set_state(self, li: int, arrays: Dict[str, np.ndarray]):
        for name, arr in arrays.items():
            if name in self.state[li]:
                dst = self.state[li][name]
                dst.copy_(torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(self.dev).reshape(dst.shape))

    def get_state(self, li: int) -> Dict[str, np.ndarray]:
        return {k: to_numpy(v) for k, v in self.state[li].items()}

    def use_inputs(self, slot: int):
        if slot != self.active:
            self.active = slot
            self._build_desc()

    # -- the step ---------------------------------------------------------
    def step(self, hp: HParams, stream=None):
        if self.mode == MODE_FULL:
            step_full(self.desc, hp, self.ws_ptr, self.ws_bytes, stream)
        else:
            step_diag(self.desc, hp, self.ws_ptr, self.ws_bytes, stream)

    def flags(self, clear: bool = False) -> int:
        return read_flags(self.ws_ptr, clear)

    @staticmethod
    def hparams(cfg_hp: Dict[str, float], refresh=True, phase_mask: int = 0) -> HParams:
        """refresh: True / False, KFAC_REFRESH_* bits, or a pair (A, G) of bools."""
        if isinstance(refresh, tuple):
            refresh = (REFRESH_A if refresh[0] else 0) | (REFRESH_G if refresh[1] else 0)
        return hparams(cfg_hp["lr"], cfg_hp["momentum"], cfg_hp["weight_decay"], cfg_hp["ema_decay"],
                       cfg_hp["damping"], refresh, phase_mask, damping_bn=cfg_hp.get("damping_bn"),
                       rescale_eps=cfg_hp.get("rescale_eps", 1e-9),
                       options=OPT_RESCALE if cfg_hp.get("rescale") else 0)
