"""MI355X-native fused clip + AdamW optimizer step (somaopt).

The compute path is the C-ABI library ``libsomaopt.so`` built from ``csrc/``
(hand-written HIP kernels for gfx950).  ``somaopt`` is its thin ctypes binding;
``workloads`` holds the seeded synthetic inputs.  Importing this package does
not load the library; ``somaopt.load()`` does, and fails loudly if it is not
built.
"""
__all__ = ["somaopt", "workloads"]
