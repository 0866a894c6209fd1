"""W4A16 linear layer for AMD Instinct MI355X (gfx950).

The compute path is ``libw4a16.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/w4a16.h``); ``weight_only_int4_gemv_amd.w4a16`` is its
thin ctypes binding.  Importing this package loads nothing; the library is
loaded on the first call and a missing library is an error, never a fallback.
"""
