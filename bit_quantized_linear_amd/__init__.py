"""MI355X (gfx950) SVDQuant W4A4 and INT8 tensorwise W8A8 linears.

The compute lives in the HIP/C++ shared library ``libsvdq.so`` built from
``csrc/`` (its C interface is ``include/svdq.h``). ``binding`` is a thin
ctypes layer with the same entry-point names that marshals numpy arrays,
torch tensors and streams into that interface; it never computes anything
itself and raises if the library is missing. ``workloads`` draws the seeded
synthetic inputs.
"""

from . import binding, workloads  # noqa: F401

__all__ = ["binding", "workloads"]
