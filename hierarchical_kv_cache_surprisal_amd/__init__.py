"""SeKV mixed-resolution decode attention and prefill builder for AMD MI355X (gfx950).

The compute path is the HIP library libsekv.so (C ABI in include/sekv.h);
`sekv` is its thin ctypes binding.
"""
from . import sekv  # noqa: F401
from .sekv import Context, SekvError, load_library  # noqa: F401
