"""Block-sparse causal attention for long-context inference on AMD MI355X (gfx950).

The compute path is libspot.so (hand-written HIP kernels behind a C ABI,
declared in include/spot.h); `block_sparse_attention_amd.binding` is its thin
ctypes wrapper and `block_sparse_attention_amd.inputs` holds the seeded
synthetic workloads.
"""
