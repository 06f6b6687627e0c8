"""SMC-SD round hot path for AMD MI355X (gfx950).

The compute lives in ``libsmcsd.so`` (hand-written HIP kernels behind a C ABI, declared in
``include/smcsd.h``); ``smc_particle_resampling_amd.smcsd`` is the thin ctypes binding with
the same names. Importing this package does not load the library; the binding does, and
raises if it is missing. ``synth`` draws seeded synthetic inputs.
"""
__all__ = ["smcsd", "synth"]


def __getattr__(name):
    if name in ("smcsd", "synth"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
