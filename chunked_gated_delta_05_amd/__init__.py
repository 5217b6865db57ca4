"""Chunkwise gated delta rule forward for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libgdn.so`` built from ``csrc/``; the
Python module ``binding`` marshals torch tensors into its C ABI (declared in
``include/gdn.h``). Importing this package does not load the library; the
first call through ``binding`` does, and fails loudly when it is missing.
"""
__all__ = ["binding", "workloads"]
