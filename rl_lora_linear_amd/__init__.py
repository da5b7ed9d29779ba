"""MI355X-native mixed-adapter LoRA training hot path.

The compute lives in the gfx950 HIP library liblora_mi355x.so (C ABI in
include/lora_mi355x.h); `rl_lora_linear_amd.lib` is its ctypes binding.  Build
the library with `python -m rl_lora_linear_amd.build`.  Importing the package
does not load the library; importing `.lib` does, and fails loudly if it is
absent.
"""
__all__ = ["build", "lib"]


def __getattr__(name):
    import importlib
    if name in ("lib", "build"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
