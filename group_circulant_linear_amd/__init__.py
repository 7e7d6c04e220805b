"""MI355X (gfx950) p4 group-circulant linear layer ("Flash EQ-Linear").

    from group_circulant_linear_amd import eqlin_prepare_weights, eqlin_forward, eqlin_backward

The compute runs in the in-tree HIP library lib/libeqlin.so (C ABI in
include/eqlin.h); `eqlin` is its thin ctypes binding and `inputs` the seeded
synthetic input generator.  Submodules load lazily so that importing the
input generator does not load the library.
"""
import importlib

_BINDING = {
    "eqlin_prepare_weights", "eqlin_forward", "eqlin_forward_ex", "eqlin_backward", "eqlin_backward_dx",
    "eqlin_backward_dw", "eqlin_prepared_weight_bytes", "eqlin_prepared_transpose_offset",
    "eqlin_backward_workspace_bytes", "load_library", "Prepared", "EqlinError",
}


def __getattr__(name):
    if name in _BINDING:
        return getattr(importlib.import_module(".eqlin", __name__), name)
    if name in ("FlashEQLinear", "EQLinearFunction", "convert_state_dict"):
        return getattr(importlib.import_module(".module", __name__), name)
    if name in ("eqlin", "inputs", "build", "module"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)


def __dir__():
    return sorted(list(_BINDING) + ["eqlin", "inputs", "build", "module", "FlashEQLinear", "EQLinearFunction"])
