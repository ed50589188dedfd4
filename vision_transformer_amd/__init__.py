"""MI355X-native (gfx950) ViT encoder forward: HIP kernels behind a C ABI.

The compute path lives in the shared library built from csrc/ (see build.py);
vitenc.py is its thin ctypes binding.  Importing this package loads nothing:
the library is opened on first use and a missing library is an error.
"""
__all__ = ["workloads"]
