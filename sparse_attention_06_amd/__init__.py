"""DeepSeek Sparse Attention hot path for MI355X (gfx950).

The compute lives in ``libdsa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/dsa.h``). ``sparse_attention_06_amd.dsa`` is the thin
ctypes binding; ``sparse_attention_06_amd.inputs`` draws the seeded synthetic
inputs. Importing the package loads neither.
"""
__all__ = ["dsa", "inputs"]
