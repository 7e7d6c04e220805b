"""Drop-in module for a group-circulant (EQ-)linear layer (p4 rotations or C8).

The Flash EQ-Linear summary (gist.science 2607.21271, "Implementation", last
bullet) describes the method as a training-free, plug-and-play replacement:
the naive layer's learnable parameters are reused unchanged.  FlashEQLinear
holds exactly those parameters, w [D/T][C/T][T], and runs the forward and
backward through the HIP library (eqlin_prepare_weights / eqlin_forward /
eqlin_backward).  The prepared spectra are cached per weight version, so they
are recomputed only after w changes (an optimizer step or a load).

There is no CPU or eager fallback: tensors must live on the GPU.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import eqlin

T_P4 = 4
GROUP_ORDERS = (4, 8)


class _SpectraCache:
    """Prepared spectra of one weight tensor, keyed on its storage and version."""

    def __init__(self):
        self.key = None
        self.prepared: Optional[eqlin.Prepared] = None

    def get(self, w: torch.Tensor) -> eqlin.Prepared:
        key = (w.data_ptr(), w._version, tuple(w.shape), w.dtype, w.device)
        if self.key != key or self.prepared is None:
            self.prepared = eqlin.eqlin_prepare_weights(w.detach().contiguous())
            self.key = key
        return self.prepared


class EQLinearFunction(torch.autograd.Function):
    """Y = X W^T with W the group-circulant expansion of w; X [..., C] -> Y [..., D]."""

    @staticmethod
    def forward(ctx, X: torch.Tensor, w: torch.Tensor, cache: Optional[_SpectraCache] = None):
        if X.dtype != w.dtype:
            raise TypeError(f"X ({X.dtype}) and w ({w.dtype}) must share a dtype")
        prepared = cache.get(w) if cache is not None else eqlin.eqlin_prepare_weights(w.detach().contiguous())
        lead = X.shape[:-1]
        X2 = X.reshape(-1, X.shape[-1]).contiguous()
        Y = eqlin.eqlin_forward(X2, prepared)
        ctx.save_for_backward(X2, w)
        ctx.prepared = prepared
        ctx.lead = lead
        return Y.reshape(*lead, prepared.D)

    @staticmethod
    def backward(ctx, dY: torch.Tensor):
        X2, w = ctx.saved_tensors
        prepared = ctx.prepared
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_dx or need_dw):
            return None, None, None
        dY2 = dY.reshape(-1, prepared.D).contiguous().to(X2.dtype)
        dX, dw = eqlin.eqlin_backward(dY2, X2 if need_dw else None, prepared, need_dx=need_dx, need_dw=need_dw)
        dX = dX.reshape(*ctx.lead, prepared.C) if dX is not None else None
        dw = dw.to(w.dtype) if dw is not None else None
        return dX, dw, None


class FlashEQLinear(torch.nn.Module):
    """Group-circulant linear layer (no bias), in_features -> out_features.

    ``group_size`` T is 4 (the p4 rotation group, the default) or 8 (C8).
    Parameter ``w`` has shape [out_features/T, in_features/T, T]; block
    (d', c') of the dense weight is the T x T circulant
    W[T d'+t, T c'+s] = w[d', c', (t - s) mod T].
    """

    def __init__(self, in_features: int, out_features: int, device=None, dtype=None, group_size: int = T_P4):
        super().__init__()
        if group_size not in GROUP_ORDERS:
            raise ValueError(f"group_size must be one of {GROUP_ORDERS}")
        T = group_size
        if in_features % T or out_features % T:
            raise ValueError(f"in_features and out_features must be multiples of {T}")
        self.in_features = in_features
        self.out_features = out_features
        self.group_size = T
        self.w = torch.nn.Parameter(torch.empty(out_features // T, in_features // T, T,
                                                device=device, dtype=dtype))
        self._cache = _SpectraCache()
        self.reset_parameters()

    def reset_parameters(self) -> None:
        # same variance per output as a dense layer of fan-in C
        torch.nn.init.normal_(self.w, 0.0, 1.0 / math.sqrt(self.in_features))

    @classmethod
    def from_naive(cls, w: torch.Tensor) -> "FlashEQLinear":
        """Wrap a naive EQ-Linear's circulant parameter w [D/T][C/T][T] (copied)."""
        Dp, Cp, T = w.shape
        if T not in GROUP_ORDERS:
            raise ValueError(f"group size {T} is not supported (use one of {GROUP_ORDERS})")
        m = cls(T * Cp, T * Dp, device=w.device, dtype=w.dtype, group_size=T)
        with torch.no_grad():
            m.w.copy_(w)
        return m

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        return EQLinearFunction.apply(X, self.w, self._cache)

    def dense_weight(self) -> torch.Tensor:
        """The expanded D x C weight (for inspection; the forward never builds it)."""
        T = self.group_size
        t = torch.arange(T, device=self.w.device)
        idx = (t.view(T, 1) - t.view(1, T)) % T
        Dp, Cp, _ = self.w.shape
        return self.w[:, :, idx].permute(0, 2, 1, 3).reshape(Dp * T, Cp * T)

    def extra_repr(self) -> str:
        group = "p4" if self.group_size == 4 else f"C{self.group_size}"
        return f"in_features={self.in_features}, out_features={self.out_features}, group={group}"


def convert_state_dict(naive_state: dict, key_map: Optional[dict] = None) -> dict:
    """Map a naive EQ-Linear state dict to FlashEQLinear keys.

    The parameters are reused unchanged (plug-and-play); ``key_map`` renames
    the naive layer's parameter key (e.g. {"weight_vec": "w"}).
    """
    key_map = key_map or {}
    out = {}
    for k, v in naive_state.items():
        prefix, _, name = k.rpartition(".")
        new = key_map.get(name, name)
        out[f"{prefix}.{new}" if prefix else new] = v
    return out
