"""MI355X-native support-aware sparse alpha-entmax decode over a paged,
GQA-shared KV cache.

The compute path is the HIP library ``libekv.so`` (built from ``csrc/``) behind
the C ABI declared in ``include/ekv.h``; ``ekv`` is its thin ctypes binding
and ``workloads`` draws seeded synthetic inputs.  Importing the package loads
nothing; ``ekv.load()`` (or the first call) opens the library and raises if
it has not been built.
"""

__all__ = ["ekv", "workloads"]
