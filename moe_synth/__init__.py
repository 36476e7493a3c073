"""Seeded synthetic inputs for the MoE FFN layer (shared by tests, bench and
the oracle's test cases; contains no arithmetic of the layer itself)."""
from .configs import (MoeConfig, CONFIGS, CONFIG_ORDER, WF_F32, WF_BF16, WF_U4,
                      ACT_SILU, ACT_GELU_TANH, DT_F32, DT_BF16, BIAS_NONE,
                      BIAS_ZIPF)
from .generator import (MoeInputs, U4Weights, generate, x_rows,
                        router_bias_values, norm_weight_values, expert_scale_values,
                        residual_values, grad_inputs,
                        f32_to_bf16_bits, f32_to_f16_bits,
                        normal_np, normal_torch, codes_np, codes_torch,
                        stream_key, tied_router_inputs)
