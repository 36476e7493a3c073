"""CPU oracle of the MoE FFN layer -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does.
"""
from . import moe_oracle
from .moe_oracle import (router_logits, softmax_row, topk_stable_desc, route,
                         permutation, expert_ffn, shared_expert, moe_ffn,
                         silu, gelu_tanh, sigmoid, bf16_to_f64, f16_to_f64,
                         u4_dequant, WeightSource, weighted_sum_backward, glu_backward,
                         rms_norm)
