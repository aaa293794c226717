"""MoEBlaze-style single-layer MoE training hot path on AMD MI355X (gfx950).

The compute lives in a HIP shared library (libmoe_dispatch.so, built from
csrc/) behind a C ABI declared in include/moe_dispatch.h.  The binding in
``binding.py`` only marshals arguments; it is imported lazily so that the
seeded workloads can be used on hosts where the library is not built.
"""

_BINDING_NAMES = {
    "moe_dispatch_build", "moe_ffn_forward", "moe_ffn_backward", "moe_last_error",
    "Shape", "MoEError", "load_library", "MOE_F32", "MOE_BF16", "MOE_SILU", "MOE_SWIGLU",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
