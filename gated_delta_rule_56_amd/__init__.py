"""Gated delta rule (GatedDeltaNet) scan for AMD MI355X (gfx950).

The compute path is libgdn.so (C ABI in include/gdn.h, HIP kernels in csrc/);
``prefill``, ``prefill_varlen``, ``decode``, ``kda_prefill``, ``kda_decode``, ``gated_rmsnorm``
and ``qkv_prologue`` are its thin torch bindings. ``inputs`` holds the seeded synthetic input generator shared with the
tests and the benchmark.
"""
from . import inputs  # noqa: F401


def __getattr__(name):
    # The binding imports torch; load it on first use so that the input
    # generator stays importable without it.
    if name in ("prefill", "prefill_varlen", "decode", "kda_prefill", "kda_decode", "gated_rmsnorm",
                "qkv_prologue", "load_library", "GdnError", "binding"):
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
