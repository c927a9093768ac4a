"""The oracle: a plain, slow, obviously correct CPU implementation of the MoE
layer forward in float64 (numpy), written from the pages that describe the
method.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or call anything in this package.  The GPU library
never routes through it, and it shares no code with the HIP path: its only
common ground with that path is the seeded input generator in ``moe_inputs``.

Every function is pinned by the CPU tests (brute force on tiny inputs, closed
forms, invariants, library routines); see ``tests/test_oracle_pins.py``.
The one reading that no test can pin is the renormalisation/scale choice of
the zero-computation-expert workload (parity unpinned: the pages print no
values for it).
"""
from .codecs import bf16_to_f64, e4m3_decode, e4m3_encode, f32_to_bf16, f64_to_bf16  # noqa: F401
from .moe import (  # noqa: F401
    MoeConfig,
    OracleResult,
    dequant_blocks,
    dequant_rows,
    down_bf16,
    down_fp8,
    gate_up_bf16,
    gate_up_fp8,
    moe_forward,
    quantize_fp8_groups,
    router_logits,
    routing_weights,
    scores,
    select_topk,
    silu,
    sort_by_expert,
    swiglu_expert_bf16,
    swiglu_expert_fp8,
)
