"""fp64 CPU oracle of the DSpark draft-round hot path.

Test infrastructure only: used by the tests, the build entry point's smoke
check and the benchmark's CPU-baseline leg, never by the product path.
"""
from .dspark_oracle import (  # noqa: F401
    NEAR_TIE, QK8_0, StepResult, attention_ragged, bf16_to_f64, conf_probe, draft_block_forward, draft_forward, draft_round, draft_round_q8, fp16_to_f64, gemv, gemv_q8,
    gemv_q8_rows, gemv_rows, greedy_argmax, lm_head, markov_sample, markov_sample_q8, markov_scores,
    markov_step, proj_smallm, q8_0_to_f64, rmsnorm, silu_gate,
)
