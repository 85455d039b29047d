"""librola: RoLA attention (block-sparse softmax + rotary low-rank linear branch) for MI355X.

The compute path is the HIP library ``librola.so`` built from ``csrc/``; the
Python module ``sparse_rank_attention_amd.rola`` only marshals arguments to it.
Importing this package does not load the library.
"""
__all__ = ["rola", "workloads"]
