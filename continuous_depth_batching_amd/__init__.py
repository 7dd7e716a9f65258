"""MI355X-native hot path of continuous depth batching (CDB).

The compute path is libcdb.so (hand-written gfx950 HIP kernels behind the C
ABI of include/cdb.h); ``_lib`` is its ctypes binding and ``engine`` holds
the device buffers and the CPU stage scheduler.  Importing ``engine``
requires the built library and raises otherwise — there is no fallback.
"""
__all__ = ["build", "engine"]
