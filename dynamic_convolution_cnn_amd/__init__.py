"""MI355X-native CondConv-style dynamic convolution.

The compute path is a HIP library for gfx950 (``csrc/``) behind a C ABI
(``include/dynconv.h``); ``binding`` is a thin ctypes layer over it that
takes torch tensors for device memory and streams. The binding loads the
library on first use and raises if it is missing: there is no CPU fallback.
"""
