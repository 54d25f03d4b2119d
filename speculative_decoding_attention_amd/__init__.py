"""MI355X-native split-KV target-verify attention (speculative decoding, topk = 1).

The product is the C-ABI library ``libverify_attn.so`` built from the HIP
sources in ``csrc/``; ``verify_attn`` is its thin ctypes binding.  Importing
this package does not load the library; importing ``verify_attn`` does, and
raises if the library has not been built.
"""

__all__ = ["verify_attn", "workloads"]
