"""Ozaki Scheme II FP64 GEMM emulation for AMD MI355X (gfx950).

The compute path is the HIP library ``liboz2.so`` (sources in ``csrc/``, C ABI in
``include/oz2.h``); ``binding`` is its thin ctypes binding.  The binding is loaded
lazily on first attribute access so that ``workloads`` (seeded inputs) and the build
driver import without a built library; any use of the compute API without the
library raises ImportError.
"""
from __future__ import annotations

import importlib

_BINDING_NAMES = {
    "ozaki2_dgemm", "ozaki2_dgemm_debug", "ozaki2_workspace_size", "ozaki2_set_workspace",
    "ozaki2_release", "ozaki2_timing_begin", "ozaki2_timing_end", "ozaki2_get_flags",
    "ozaki2_moduli", "ozaki2_tau", "ozaki2_status_string", "dgemm", "dgemm_debug",
    "colmajor", "empty_colmajor", "Oz2Error", "OZ2Dump", "OZ2_FAST", "OZ2_ACCU", "OZ2_OK",
    "OZ2_ERR_ARG", "OZ2_ERR_UNSUPPORTED", "OZ2_ERR_WORKSPACE", "OZ2_ERR_HIP",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        mod = importlib.import_module(".binding", __name__)
        return getattr(mod, name)
    raise AttributeError(name)
