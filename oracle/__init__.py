"""fp64 CPU oracle of the LAGA per-rank attention path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from .laga_oracle import (  # noqa: F401
    absorbed_backward,
    absorbed_forward_rows,
    absorbed_scores_and_out,
    attention_bwd,
    attention_fwd,
    attention_fwd_rows,
    backward,
    explicit_scores,
    forward,
    head_shard,
    kv_up,
    kv_up_bwd,
    latent_rmsnorm,
    latent_rmsnorm_bwd,
)
