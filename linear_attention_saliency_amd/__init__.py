"""MI355X-native STILL hybrid attention layer (HIP kernels behind a C ABI).

The ctypes binding lives in `linear_attention_saliency_amd.still`; importing this package
does not load the native library.
"""
