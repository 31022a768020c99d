"""fp64 CPU oracle of the fused clip + AdamW optimizer step.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product library or its binding.
"""
from .adamw_fp64 import (CLIP_EPS, Group, Oracle, StepStats, adamw_update,  # noqa: F401
                         clip_coefficient, global_norm, normalized_sumsq,
                         round_to_bf16_bits, round_to_f16, update_elements, widen_grad)
from .attention_fp64 import (attention_backward, attention_forward, attention_probs,  # noqa: F401
                             error_budget_backward, error_budget_forward)
from .accumulate_fp64 import accumulate_gradient  # noqa: F401
from .schedule_fp64 import scheduled_lr  # noqa: F401
