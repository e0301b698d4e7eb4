"""MI355X-native forward pass of a non-causal multi-head self-attention block.

The compute lives in ``libattnblock.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/attn_block.h``); ``binding`` marshals torch
tensors and streams into those calls. Importing this package does not load the
library; ``binding.lib()`` does, and raises if it is missing.
"""
