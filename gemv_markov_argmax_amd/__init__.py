"""DSpark draft-round hot path on AMD Instinct MI355X (gfx950).

The compute lives in libdspark.so (hand-written HIP kernels behind a C ABI,
declared in include/dspark.h); ``ops`` is a thin ctypes binding with the same
entry-point names. ``synth`` draws the seeded synthetic inputs.
"""

__all__ = ["ops", "synth", "build"]


def __getattr__(name):  # lazy: importing the package loads neither torch nor the library
    if name in ("ops", "synth", "build"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
