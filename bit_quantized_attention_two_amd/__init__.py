"""MiniKV-style compressed-KV attention for MI355X (gfx950).

The compute path is the HIP library ``libminikv.so`` (hand-written kernels
behind a C ABI, declared in ``include/minikv.h``).  ``minikv`` is its thin
ctypes binding; ``configs`` and ``synth`` describe and draw the synthetic
workloads.  The binding is imported lazily so that the pure-Python modules
stay usable on hosts without a GPU.
"""
__all__ = ["configs", "synth", "minikv"]
__version__ = "0.1.0"


def __getattr__(name):
    if name == "minikv":
        import importlib
        return importlib.import_module(__name__ + ".minikv")
    raise AttributeError(name)
