"""CPU oracle for the Q4 expert path: gate/up + SwiGLU, down, whole expert (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP path.
"""
from .q4_oracle import (  # noqa: F401
    OFFSET_ABSENT,
    bf16_to_f32,
    f32_to_bf16,
    f32_round_dyadic,
    f32_parts,
    check_layout,
    q4_weights,
    q8_weights,
    weight_bytes,
    row_scales,
    exact_dots,
    scaled_f32,
    swiglu_tail,
    swiglu_tail_f32,
    f32_integer_parts,
    expert_gate_up,
    expert_gate_up_grouped,
    check_down_layout,
    expert_down,
    expert_forward,
    expert_down_grouped,
    expert_forward_grouped,
)
