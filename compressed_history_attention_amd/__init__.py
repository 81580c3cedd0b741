"""libnanokv: compressed-history attention (NanoKV) on AMD Instinct MI355X.

The compute path is the HIP library ``libnanokv.so`` built from ``csrc/``;
``lib`` is its thin ctypes binding and ``synth`` draws seeded workloads.
Importing the package does not load the library; the first call into
``lib`` does, and raises if it has not been built.
"""
__all__ = ["lib", "synth"]
