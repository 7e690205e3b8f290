"""MI355X-native Mamba-3 SSM layer core.

The compute lives in hand-written gfx950 HIP kernels behind the C ABI declared
in ``include/mamba3_ssm.h`` (shared library ``libmamba3_ssm.so`` in this
package directory).  ``state_space_sequence_03_amd.ops`` is a thin ctypes
binding with the same entry-point names; it marshals torch tensors (device
memory and streams only) and raises if the library is missing.
"""
import importlib

__all__ = ["ops", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
