"""CPU oracle for the masked-token readout of a masked diffusion LLM.

TEST INFRASTRUCTURE ONLY.  Plain, slow, fp64 NumPy code written from the
pages' definitions; only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library (``masked_token_logits_amd``) and neither imports the other.
"""
from .readout import (  # noqa: F401
    widen_bf16,
    candidate_positions,
    logits,
    row_stats,
    select_topk,
    select_threshold,
    apply_updates,
    readout_step,
    readout_step_batch,
    readout_rows,
    StepResult,
)
from .ffn import silu, ffn_rows, ffn_chunked  # noqa: F401,E402
