"""libkvmem: IndexMem / MomentKV KV-cache eviction hot path for AMD MI355X (gfx950).

The compute lives in the HIP library libkvmem.so (include/kvm.h); this package is its
torch-facing binding.  Importing it loads the library and fails if it is not built.
"""
from ._lib import KvmError, lib  # noqa: F401
from .api import *  # noqa: F401,F403

lib()
