"""MI355X (gfx950) group-circulant linear layer ("Flash EQ-Linear") for the
groups p4, C8 and p4m, and the p4 group convolution built on it.

    from group_circulant_linear_amd import eqlin_prepare_weights, eqlin_forward, eqlin_backward
    from group_circulant_linear_amd import FlashEQLinear, FlashEQConv2d

The compute runs in the in-tree HIP library lib/libeqlin.so (C ABI in
include/eqlin.h and include/eqconv.h); `eqlin` is its thin ctypes binding and
`inputs` the seeded synthetic input generator.  Submodules load lazily so
that importing the input generator does not load the library.
"""
import importlib

_BINDING = {
    "eqlin_prepare_weights", "eqlin_forward", "eqlin_forward_ex", "eqlin_forward_plan", "eqlin_backward", "eqlin_backward_dx",
    "eqlin_backward_dw", "eqlin_prepared_weight_bytes", "eqlin_prepared_transpose_offset",
    "eqlin_backward_workspace_bytes", "load_library", "Prepared", "EqlinError",
    "eqconv_prepare_weights", "eqconv_forward", "eqconv_backward", "eqconv_prepared_weight_bytes",
    "eqconv_backward_workspace_bytes", "ConvPrepared",
}
_MODULE = {"FlashEQLinear", "EQLinearFunction", "convert_state_dict", "FlashEQConv2d", "EQConvFunction"}


def __getattr__(name):
    if name in _BINDING:
        return getattr(importlib.import_module(".eqlin", __name__), name)
    if name in _MODULE:
        return getattr(importlib.import_module(".module", __name__), name)
    if name in ("eqlin", "inputs", "build", "module"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)


def __dir__():
    return sorted(list(_BINDING) + list(_MODULE) + ["eqlin", "inputs", "build", "module"])
