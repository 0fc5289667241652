"""MI355X-native hot path of Heterogeneous Step Allocation (HSA) for
flow-matching DiT video sampling: a C-ABI HIP library (libhsa.so, gfx950) and
its Python binding.  See include/hsa.h for the entry points."""
from . import hsa  # noqa: F401

__all__ = ["hsa"]
