"""MI355X-native AWQ per-layer activation-aware scale search.

The compute path is the C-ABI library libawq.so (hand-written HIP kernels for
gfx950) declared in include/awq.h; `awq` is its thin Python binding over torch
device tensors and `synth` draws the seeded synthetic layers.
"""
__all__ = ["awq", "synth"]
