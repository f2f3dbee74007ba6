"""KDA (Kimi Delta Attention) prefill for MI355X (gfx950).

The computation lives in libkda.so (HIP kernels behind the C ABI in
include/kda.h); `gated_delta_rule_46_amd.kda` is its Python binding.  The
binding is imported lazily so that `gated_delta_rule_46_amd.build` works
before the library exists.
"""
import importlib

__all__ = ["kda", "build"]


def __getattr__(name):
    if name in ("kda", "build"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
