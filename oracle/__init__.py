"""CPU float64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library and its Python binding
never call it: there is no CPU fallback.  It shares no code with the HIP
path; the two meet only in the seeded input generators of
``exact_attention_88_amd.workloads``, which hold no attention arithmetic.
"""
from .attention import (attention_forward, attention_backward, delta_rowsum, head_forward,
                        head_backward, head_forward_rows, head_backward_rows,
                        head_backward_qrows, causal_offset)

__all__ = ["attention_forward", "attention_backward", "delta_rowsum", "head_forward",
           "head_backward", "head_forward_rows", "head_backward_rows", "head_backward_qrows",
           "causal_offset"]
