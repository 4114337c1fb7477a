"""fp64 CPU oracle for Multi-Scale Retention (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg import this
package. It never imports the HIP library or its binding.
"""

from .retention_oracle import (  # noqa: F401
    backward,
    backward_rows,
    chunkwise,
    decay_mask,
    gated_group_norm,
    group_norm,
    group_norm_rows,
    parallel,
    parallel_rows,
    recurrent,
    recurrent_step,
    state_after,
    swish,
    xpos_rotate,
)
