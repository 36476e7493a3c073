"""Shapes and value recipes of the five synthetic MoE FFN workloads.

Each workload is a mixture-of-experts feed-forward layer (router, softmax,
top-k, renormalise, gated expert FFNs, weighted combine, optional
sigmoid-gated shared expert).  The shapes follow the pages:

* ``tiny_f32`` -- a hand-checkable f32 case (SwiGLU, 8 experts, top-2).
* ``decode_geglu_t1`` -- one token through the GELU-GLU expert shape that
  mlx-native's moe_dispatch.rs documents for MoeDispatchParams
  (input 2816, intermediate 704, 8 selected experts), 128 experts, bf16
  weights, f32 activations.
* ``prefill_shared_t4096`` -- 4096 tokens through the 256-expert,
  512-intermediate, 2048-hidden shape that hf2q's qwen35/gpu_ffn.rs sizes
  in its MoeFfnWeightsGpu memory note, with one sigmoid-gated shared
  expert, bf16 weights and activations.
* ``decode_u4_t32`` -- 32 tokens with affine 4-bit group-32 expert weights
  (w = code*scale + min), f32 activations.
* ``prefill_skew_t16384`` -- 16384 tokens, hidden 7168, intermediate 2048,
  256 experts, top-8, shared expert, with a per-expert router bias
  -2*ln(e+1) that skews the load towards low expert ids.

No method arithmetic lives here: only sizes, dtypes and distributions.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

# weight formats (same integer values as the C ABI enum)
WF_F32 = 0
WF_BF16 = 1
WF_U4 = 2

# activations
ACT_SILU = 0
ACT_GELU_TANH = 1

# activation / router storage dtypes
DT_F32 = 0
DT_BF16 = 1

# router-bias recipes
BIAS_NONE = 0
BIAS_ZIPF = 1   # b_e = -2 * ln(e + 1)


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden
    I: int                 # routed intermediate
    E: int                 # experts
    k: int                 # top-k
    act: int = ACT_SILU
    weight_format: int = WF_F32
    act_dtype: int = DT_F32
    router_dtype: int = DT_F32
    shared: bool = False
    Is: int = 0            # shared intermediate
    bias: int = BIAS_NONE
    group_size: int = 32   # u4 quantisation group along K
    seed_index: int = 0    # master seed is 0x5EED0000 + seed_index

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.seed_index

    @property
    def routes(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "MoeConfig":
        return replace(self, T=T)


CONFIGS = {
    "tiny_f32": MoeConfig(
        name="tiny_f32", T=4, H=64, I=32, E=8, k=2, act=ACT_SILU,
        weight_format=WF_F32, act_dtype=DT_F32, router_dtype=DT_F32,
        seed_index=0),
    "decode_geglu_t1": MoeConfig(
        name="decode_geglu_t1", T=1, H=2816, I=704, E=128, k=8,
        act=ACT_GELU_TANH, weight_format=WF_BF16, act_dtype=DT_F32,
        router_dtype=DT_BF16, seed_index=1),
    "prefill_shared_t4096": MoeConfig(
        name="prefill_shared_t4096", T=4096, H=2048, I=512, E=256, k=8,
        act=ACT_SILU, weight_format=WF_BF16, act_dtype=DT_BF16,
        router_dtype=DT_BF16, shared=True, Is=512, seed_index=2),
    "decode_u4_t32": MoeConfig(
        name="decode_u4_t32", T=32, H=4096, I=1536, E=128, k=8,
        act=ACT_SILU, weight_format=WF_U4, act_dtype=DT_F32,
        router_dtype=DT_F32, seed_index=3),
    "prefill_skew_t16384": MoeConfig(
        name="prefill_skew_t16384", T=16384, H=7168, I=2048, E=256, k=8,
        act=ACT_SILU, weight_format=WF_BF16, act_dtype=DT_BF16,
        router_dtype=DT_BF16, shared=True, Is=2048, bias=BIAS_ZIPF,
        seed_index=4),
}

CONFIG_ORDER = ["tiny_f32", "decode_geglu_t1", "prefill_shared_t4096",
                "decode_u4_t32", "prefill_skew_t16384"]
