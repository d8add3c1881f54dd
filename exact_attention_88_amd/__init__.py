"""Exact attention (FlashAttention-2 forward and backward) for AMD MI355X.

The compute path is the HIP library ``libfa.so`` (C ABI in ``include/fa.h``);
``exact_attention_88_amd.fa`` is its thin Python binding and
``exact_attention_88_amd.workloads`` holds the seeded synthetic inputs.
"""
__version__ = "0.1.0"
