"""Drop-in module for a group-circulant (EQ-)linear layer (p4, C8 or p4m).

The Flash EQ-Linear summary (gist.science 2607.21271, "Implementation", last
bullet) describes the method as a training-free, plug-and-play replacement:
the naive layer's learnable parameters are reused unchanged.  FlashEQLinear
holds exactly those parameters, w [D/n][C/n][n] (n = group order), and runs the forward and
backward through the HIP library (eqlin_prepare_weights / eqlin_forward /
eqlin_backward).  The prepared spectra are cached per weight version, so they
are recomputed only after w changes (an optimizer step or a load).

FlashEQConv2d does the same for the p4 group convolution with K x K filters
(the summary's "Limitations and future work" names equivariant convolution
as the next operator): parameter psi [D/4][C/4][K][K][4], channels-last maps,
forward and backward through eqconv_prepare_weights / eqconv_forward /
eqconv_backward; its 1 x 1 case is FlashEQLinear with group p4.

There is no CPU or eager fallback: tensors must live on the GPU.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import eqlin

T_P4 = 4


def cayley_table(code: int) -> torch.Tensor:
    """Multiplication table of the group (index of g_i g_j): cyclic for 4 and 8;
    for p4m the element u = k + 4m is r^k s^m with s r s = r^-1."""
    n = eqlin.group_order(code)
    i = torch.arange(n)
    if code != eqlin.EQLIN_P4M:
        return (i.view(n, 1) + i.view(1, n)) % n
    k, m = i % 4, i // 4
    k1, m1, k2, m2 = k.view(n, 1), m.view(n, 1), k.view(1, n), m.view(1, n)
    return (k1 + torch.where(m1 == 0, k2, -k2)) % 4 + 4 * (m1 ^ m2)


def dense_expansion(w: torch.Tensor, group=None) -> torch.Tensor:
    """The dense D x C weight W[n d'+g, n c'+h] = w[d', c', h^-1 g] of w [D/n][C/n][n]
    (group None: cyclic of order n).  For inspection and dense comparisons only."""
    code = eqlin.group_code(w.shape[2] if group is None else group)
    n = eqlin.group_order(code)
    table = cayley_table(code)
    inv = torch.stack([torch.nonzero(table[i] == 0)[0, 0] for i in range(n)])
    idx = table[inv.view(1, n), torch.arange(n).view(n, 1)].to(w.device)   # idx[g, h] = h^-1 g
    Dp, Cp, _ = w.shape
    return w[:, :, idx].permute(0, 2, 1, 3).reshape(Dp * n, Cp * n)


class _SpectraCache:
    """Prepared spectra of one weight tensor, keyed on its storage and version."""

    def __init__(self):
        self.key = None
        self.prepared: Optional[eqlin.Prepared] = None

    def get(self, w: torch.Tensor, group=None) -> eqlin.Prepared:
        key = (w.data_ptr(), w._version, tuple(w.shape), w.dtype, w.device, group)
        if self.key != key or self.prepared is None:
            self.prepared = eqlin.eqlin_prepare_weights(w.detach().contiguous(), group=group)
            self.key = key
        return self.prepared


class EQLinearFunction(torch.autograd.Function):
    """Y = X W^T with W the group-circulant expansion of w; X [..., C] -> Y [..., D].
    group: None (cyclic of order w.shape[2]) or a group accepted by eqlin.group_code."""

    @staticmethod
    def forward(ctx, X: torch.Tensor, w: torch.Tensor, cache: Optional[_SpectraCache] = None, group=None):
        if X.dtype != w.dtype:
            raise TypeError(f"X ({X.dtype}) and w ({w.dtype}) must share a dtype")
        prepared = (cache.get(w, group) if cache is not None
                    else eqlin.eqlin_prepare_weights(w.detach().contiguous(), group=group))
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
            return None, None, None, None
        dY2 = dY.reshape(-1, prepared.D).contiguous().to(X2.dtype)
        dX, dw = eqlin.eqlin_backward(dY2, X2 if need_dw else None, prepared, need_dx=need_dx, need_dw=need_dw)
        dX = dX.reshape(*ctx.lead, prepared.C) if dX is not None else None
        dw = dw.to(w.dtype) if dw is not None else None
        return dX, dw, None, None


class FlashEQLinear(torch.nn.Module):
    """Group-circulant linear layer (no bias), in_features -> out_features.

    ``group`` is 4 or "p4" (the p4 rotation group, the default), 8 or "c8"
    (the cyclic group C8), or "p4m" (rotations and reflections, order 8).
    Parameter ``w`` has shape [out_features/n, in_features/n, n] (n = group
    order); block (d', c') of the dense weight is W[n d'+g, n c'+h] =
    w[d', c', h^-1 g], for the cyclic groups the circulant w[d', c', (g-h) mod n].
    """

    def __init__(self, in_features: int, out_features: int, device=None, dtype=None, group=T_P4):
        super().__init__()
        code = eqlin.group_code(group)
        n = eqlin.group_order(code)
        if in_features % n or out_features % n:
            raise ValueError(f"in_features and out_features must be multiples of {n}")
        self.in_features = in_features
        self.out_features = out_features
        self.group = code
        self.group_size = n
        self.w = torch.nn.Parameter(torch.empty(out_features // n, in_features // n, n,
                                                device=device, dtype=dtype))
        self._cache = _SpectraCache()
        self.reset_parameters()

    def reset_parameters(self) -> None:
        # same variance per output as a dense layer of fan-in C
        torch.nn.init.normal_(self.w, 0.0, 1.0 / math.sqrt(self.in_features))

    @classmethod
    def from_naive(cls, w: torch.Tensor, group=None) -> "FlashEQLinear":
        """Wrap a naive EQ-Linear's parameter w [D/n][C/n][n] (copied); group None
        means the cyclic group of order n = w.shape[2]."""
        Dp, Cp, n = w.shape
        code = eqlin.group_code(n if group is None else group)
        if eqlin.group_order(code) != n:
            raise ValueError(f"w's last dimension {n} is not the order of group {group!r}")
        m = cls(n * Cp, n * Dp, device=w.device, dtype=w.dtype, group=code)
        with torch.no_grad():
            m.w.copy_(w)
        return m

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        return EQLinearFunction.apply(X, self.w, self._cache, self.group)

    def dense_weight(self) -> torch.Tensor:
        """The expanded D x C weight (for inspection; the forward never builds it)."""
        return dense_expansion(self.w, self.group)

    def extra_repr(self) -> str:
        group = {4: "p4", 8: "C8", eqlin.EQLIN_P4M: "p4m"}[self.group]
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


# ------------------------------------------------------------ p4 group convolution

def conv_dense_filter(psi: torch.Tensor) -> torch.Tensor:
    """The ordinary K x K filter bank [D][C][K][K] of the p4 group convolution
    with filter psi [D/4][C/4][K][K][4]: output channel d'*4 + r, input channel
    c'*4 + s holds psi[d', c', R^-r delta, (r - s) mod 4] at tap delta, i.e.
    the filter turned r times (torch.rot90 on the tap axes).  For inspection
    and dense comparisons only; the convolution never builds it."""
    Dp, Cp, K = psi.shape[0], psi.shape[1], psi.shape[2]
    flat = torch.arange(psi.numel()).reshape(psi.shape)
    idx = torch.empty((4 * Dp, 4 * Cp, K, K), dtype=torch.long)
    for r in range(4):
        turned = torch.rot90(flat, r, dims=(2, 3))
        for s in range(4):
            idx[r::4, s::4] = turned[..., (r - s) % 4]
    return psi.reshape(-1)[idx.to(psi.device)]


class _ConvSpectraCache:
    """Prepared filter spectra of one filter tensor, keyed on its storage and version."""

    def __init__(self):
        self.key = None
        self.prepared: Optional[eqlin.ConvPrepared] = None

    def get(self, psi: torch.Tensor) -> eqlin.ConvPrepared:
        key = (psi.data_ptr(), psi._version, tuple(psi.shape), psi.dtype, psi.device)
        if self.key != key or self.prepared is None:
            self.prepared = eqlin.eqconv_prepare_weights(psi.detach().contiguous())
            self.key = key
        return self.prepared


class EQConvFunction(torch.autograd.Function):
    """p4 group convolution, X [N][H][W][C] -> Y [N][H][W][D] (channels last,
    rotation fastest), optional group-invariant bias and GELU (forward only)."""

    @staticmethod
    def forward(ctx, X: torch.Tensor, psi: torch.Tensor, cache: Optional[_ConvSpectraCache] = None):
        if X.dtype != psi.dtype:
            raise TypeError(f"X ({X.dtype}) and psi ({psi.dtype}) must share a dtype")
        prepared = cache.get(psi) if cache is not None else eqlin.eqconv_prepare_weights(psi.detach().contiguous())
        Xc = X.contiguous()
        Y = eqlin.eqconv_forward(Xc, prepared)
        ctx.save_for_backward(Xc, psi)
        ctx.prepared = prepared
        return Y

    @staticmethod
    def backward(ctx, dY: torch.Tensor):
        X, psi = ctx.saved_tensors
        need_dx, need_dpsi = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_dx or need_dpsi):
            return None, None, None
        dX, dpsi = eqlin.eqconv_backward(dY.contiguous().to(X.dtype), X if need_dpsi else None, ctx.prepared,
                                         need_dx=need_dx, need_dpsi=need_dpsi)
        return dX, (dpsi.to(psi.dtype) if dpsi is not None else None), None


class FlashEQConv2d(torch.nn.Module):
    """p4 group convolution of regular feature maps (the 1 x 1 case is FlashEQLinear).

    Input and output are channels-last maps [N][H][W][C] with channel
    c'*4 + s (rotation s fastest); ``kernel_size`` K is odd and the padding
    keeps the image size.  Parameter ``psi`` [out/4][in/4][K][K][4]:
    Y[x, d'*4 + r] = sum X[x + delta, c'*4 + s] psi[d', c', R^-r delta, (r - s) mod 4]
    with R the quarter turn of the pixel grid.
    """

    def __init__(self, in_channels: int, out_channels: int, kernel_size: int = 3, device=None, dtype=None):
        super().__init__()
        if in_channels % 4 or out_channels % 4:
            raise ValueError("in_channels and out_channels must be multiples of 4")
        if kernel_size % 2 != 1:
            raise ValueError("kernel_size must be odd")
        self.in_channels = in_channels
        self.out_channels = out_channels
        self.kernel_size = kernel_size
        self.psi = torch.nn.Parameter(torch.empty(out_channels // 4, in_channels // 4, kernel_size, kernel_size, 4,
                                                  device=device, dtype=dtype))
        self._cache = _ConvSpectraCache()
        self.reset_parameters()

    def reset_parameters(self) -> None:
        torch.nn.init.normal_(self.psi, 0.0, 1.0 / math.sqrt(self.in_channels * self.kernel_size ** 2))

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        return EQConvFunction.apply(X, self.psi, self._cache)

    def extra_repr(self) -> str:
        return f"in_channels={self.in_channels}, out_channels={self.out_channels}, kernel_size={self.kernel_size}, group=p4"
