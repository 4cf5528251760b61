"""MI355X-native paged KV cache attention.

The compute path lives in libpagedkv.so (hand-written HIP kernels for gfx950
behind a C ABI declared in include/pagedkv.h).  `pagedkv` is the thin ctypes
binding; `workloads` builds seeded synthetic inputs.  Importing this package
does not load the library; the first call into `pagedkv` does, and raises if
it has not been built.
"""
__all__ = ["pagedkv", "workloads"]
