"""CPU oracle for exact multi-head softmax attention (test infrastructure).

This package is test infrastructure only. The tests, the smoke check and
the CPU-baseline leg of the benchmark may import it; the library and its
Python binding never do, and the HIP path shares no code with it.

Every function computes in float64 with plain numpy: the definition of
the operation written out, with no blocking beyond independent query-row
blocks, no fusion and no reordering of the mathematics.
"""
from .attention import (attention_ref, merge_ref, permute_ref,
                        inverse_permute_ref, attention_flops, attention_bwd_ref)

__all__ = ["attention_ref", "merge_ref", "permute_ref", "inverse_permute_ref",
           "attention_flops", "attention_bwd_ref"]
