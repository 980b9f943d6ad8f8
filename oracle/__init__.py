"""fp64 CPU oracle for multi-scale retention (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  See ``retention_oracle`` for what it computes.
"""
from .retention_oracle import (chunk_state_contribution, chunkwise, group_norm, parallel, recurrent,
                               recurrent_backward, recurrent_step)

__all__ = ["recurrent", "recurrent_step", "parallel", "chunkwise", "chunk_state_contribution",
           "recurrent_backward", "group_norm"]
