"""MI355X-native SPRINT block step: HIP kernels behind a C ABI (libsprint.so).

The binding is in :mod:`sparse_prefix_kv_amd.sprint`; the seeded synthetic
inputs are in :mod:`sparse_prefix_kv_amd.synth`.  Importing the package does
not load the library; the first call does, and raises if it is not built.
"""
