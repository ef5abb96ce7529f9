"""fp64 CPU oracle for exact softmax attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package; the HIP library and its binding never do.
"""
from .attention import (brute_fwd, head_bwd, head_chunked_bwd,
                        head_chunked_fwd, head_fwd, head_lse, head_scores,
                        lse_merge, ref_bwd, ref_fwd, stack_bwd, stack_fwd)

__all__ = ["brute_fwd", "head_bwd", "head_chunked_bwd", "head_chunked_fwd",
           "head_fwd", "head_lse", "head_scores", "lse_merge", "ref_bwd",
           "ref_fwd", "stack_bwd", "stack_fwd"]
