"""Ternary-weight FP16 GEMV/GEMM (TQ2 / TQ1 packings) for MI355X (gfx950).

The compute lives in libtq.so (C ABI in include/tq.h); ``binding`` exposes its
entry points under the same names.  Importing the package itself does not load
the library, so the build step can run first; touching any binding name loads
it and fails loudly if it has not been built.
"""

__all__ = ["binding"]


def __getattr__(name):
    import importlib
    if name.startswith("__"):
        raise AttributeError(name)
    if name in ("binding", "build_lib"):
        # submodules: resolving build_lib must not load the library it rebuilds
        return importlib.import_module(__name__ + "." + name)
    binding = importlib.import_module(__name__ + ".binding")
    return getattr(binding, name)
