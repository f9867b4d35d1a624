"""Packed 4-bit dequant-in-register MoE FFN and dense GEMV for MI355X (gfx950).

The compute lives in ``libdqg.so`` (HIP, built in-tree by ``dequant_gemv_amd.build``);
``dequant_gemv_amd.binding`` marshals torch tensors into its C ABI (``include/dqg.h``).
Importing the package does not load the library; importing ``binding`` does, and fails
loudly when the library has not been built.
"""
__all__ = ["binding", "build"]
