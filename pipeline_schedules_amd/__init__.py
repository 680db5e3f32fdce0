"""pipeline_schedules_amd -- a 1F1B pipeline-stage executor for MI355X (gfx950).

The compute path lives in ``libpps.so`` (C ABI declared in ``include/pps.h``;
HIP kernels under ``csrc/``).  ``pipeline_schedules_amd.pps`` is a thin ctypes
binding with the same names; it only marshals arguments.

Submodules are imported lazily so that ``configs`` and ``inputs`` (seeded
synthetic data) can be used without the native library.  Any use of the
binding raises at once if ``libpps.so`` has not been built.
"""

import importlib

__all__ = ["configs", "inputs", "pps"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
