"""Stream-Factorized Attention (Hidden Decoding) on AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libhd.so`` (C ABI in ``include/hd.h``);
``latent_sequence_length_amd.hd`` is its thin Python binding.  ``synth`` holds
the seeded synthetic input generators used by tests and the benchmark.
"""
__all__ = ["hd", "synth"]


def __getattr__(name):
    if name in ("hd", "synth", "build"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
