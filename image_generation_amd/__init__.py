"""MI355X-native DiT denoise step: HIP kernels behind a C ABI (libdit.so).

Import ``image_generation_amd.dit`` for the ctypes binding; it raises ImportError
when libdit.so has not been built.
"""
