"""MI355X-native 3D-RoPE sparse + low-rank hybrid attention forward.

The compute lives in the HIP library ``libslr.so`` (built from ``csrc/``);
``binding`` marshals torch device tensors into its C ABI. Importing this
package does not load the library; the first call through ``binding`` does,
and fails loudly if it is missing.
"""
__all__ = ["binding", "synth"]
