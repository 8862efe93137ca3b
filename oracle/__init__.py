"""CPU oracle for the MoE layer forward (test infrastructure only).

Only the tests, the package entry's smoke check and the benchmark's CPU
baseline leg may import this package.  It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (GATE_TOPK_SOFTMAX, GATE_SOFTMAX_TOPK,  # noqa: F401
                         GATE_SOFTMAX_TOPK_RENORM, GATE_SIGMOID_BIAS_RENORM, GATING_MODES)
