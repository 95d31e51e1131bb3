"""Q-GaLore optimizer step on MI355X (gfx950): Python front end of libqgalore.so.

The compute runs in the library's HIP kernels (csrc/); `binding` marshals torch tensors
across its C ABI (include/qgalore.h). `workloads` holds the seeded synthetic inputs.
Submodules are imported on first use so that the input generators load without the library.
"""
import importlib

__all__ = ["binding", "workloads", "build"]


def __getattr__(name):
    if name in ("binding", "workloads", "build"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
