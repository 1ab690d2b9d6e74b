"""libcca for AMD Instinct MI355X: the CCA / CCGQA forward pass (prefill and
one decode step) as hand-written HIP kernels behind a C ABI (include/cca.h).

    from efficient_transformer_attention_amd import cca   # ctypes binding of libcca.so
    python -m efficient_transformer_attention_amd.build     # builds libcca.so

The binding is imported on first use so that the build step can run before
the library exists; importing ``cca`` raises if libcca.so is missing.
"""

__all__ = ["cca", "tensors", "build"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
