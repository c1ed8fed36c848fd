"""R-SWA (Reference Sliding Window Attention) on AMD MI355X.

The compute path is the HIP library built from csrc/ (librswa.so) behind the
C ABI declared in include/rswa.h.  ``kv_cache_management_amd.rswa`` is the thin
ctypes binding to it; importing this package itself loads nothing.
"""
