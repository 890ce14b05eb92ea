"""Batched speculative-decoding verify on MI355X (gfx950).

The compute path is the C-ABI library ``libspecverify.so`` built from
``csrc/`` (hand-written HIP kernels); ``binding`` marshals torch tensors into
its entry points.  Importing this package does not load the library; the
first call does, and fails loudly when it is missing.
"""
__all__ = ["binding", "synth"]
