"""MI355X-native paged KV-cache attention with per-layer mask regimes.

The compute lives in libpakv.so (hand-written HIP kernels for gfx950 behind a
C ABI, declared in include/pakv.h); ``full_attention_amd.pakv`` is its thin
ctypes binding (importing it fails if the library is not built).  PyTorch is
used only for device memory and streams.
"""
