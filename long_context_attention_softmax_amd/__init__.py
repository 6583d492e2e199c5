"""Hybrid compressed attention (DeepSeek-V4 CSA + HCA) on MI355X / gfx950.

The hot path - softmax-gated KV pooling, the lightning indexer with top-k, and
shared-KV multi-query attention with one softmax over compressed entries, a
sliding window and a sink - runs in hand-written HIP kernels behind the C ABI of
``include/hca.h``.  ``ops`` is the Python boundary with the C entry-point names;
``layer.DeviceLayer`` keeps one layer's buffers resident and runs its step.

Importing ``ops`` or ``layer`` loads the built library and fails if it is missing.
"""
__all__ = ["ops", "layer"]
