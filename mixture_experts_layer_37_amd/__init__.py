"""MI355X-native forward pass of one Mixture-of-Experts layer.

The computation lives in libmoe.so (HIP kernels for gfx950 behind the C ABI of
include/moe.h); `binding` is its ctypes binding and `inputs` the seeded
synthetic workloads.  Importing the package loads nothing.
"""
