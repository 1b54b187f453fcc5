"""Modulated deformable 2-D convolution (DCNv2) forward for MI355X (gfx950).

The computation lives in libmdcn.so (C ABI in include/mdcn.h, HIP kernels in
csrc/); ``mdcn`` is its Python binding and ``workloads`` draws seeded
synthetic inputs.  Importing the package loads nothing.
"""
