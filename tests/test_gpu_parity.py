"""GPU parity: the HIP library (through the C ABI) against the float64 CPU
oracle on identical seeded inputs.  Routing ids and the expert grouping
must be bit-exact; routing weights within 1e-5; outputs within
max|GPU-CPU|/max|CPU| <= 1e-4 (f32 weights), 2e-2 (bf16), 3e-2 (4-bit)."""
import ctypes

import numpy as np
import pytest

from moe_synth import (CONFIGS, MoeConfig, WF_F32, WF_BF16, WF_U4, ACT_SILU, ACT_GELU_TANH,
                       DT_F32, DT_BF16, BIAS_ZIPF)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_ffn_gemv_amd as M
    M.load()


from parity_util import Case, check_case, log, rel_err, TOL as TOL_BY_WF  # noqa: E402

# ----------------------------------------------------------- full workloads
# Every token at the decode shapes.  At the prefill shapes, the tokens of
# route tiles spread over the grouped GEMMs' whole tile list (every XCD's
# share), the most loaded expert's ragged last tile and the shared
# expert's last tile: at least 32 tokens at 4096, 16 at 16384.
FULL_SPREAD = {
    "tiny_f32": None,
    "decode_geglu_t1": None,
    "decode_u4_t32": None,
    "prefill_shared_t4096": 32,
    "prefill_skew_t16384": 16,
}


@pytest.mark.parametrize("name", list(FULL_SPREAD))
def test_full_workload_parity(name):
    from oracle_driver import tile_covering_tokens
    cfg = CONFIGS[name]
    case = Case(cfg)
    spread = FULL_SPREAD[name]
    pick = None
    if spread:
        def pick(ids):
            return tile_covering_tokens(ids, cfg.E, cfg.k, cfg.T, cfg.shared, spread=spread)
    res = check_case(case, tokens_from_ids=pick)
    if spread:
        assert len(res["tokens"]) >= spread


# ----------------------------------------------- small shapes, every token
SMALL = [
    # MFMA path: several route tiles per expert, ragged tails, shared expert
    MoeConfig(name="mfma_shared", T=300, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=192, seed_index=11),
    MoeConfig(name="mfma_two_tiles", T=700, H=192, I=64, E=8, k=2, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=12),
    MoeConfig(name="mfma_gelu_bias", T=257, H=128, I=192, E=32, k=8, act=ACT_GELU_TANH,
              weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, bias=BIAS_ZIPF,
              shared=True, Is=64, seed_index=13),
    # 256-route tiles with direct-to-LDS operand loads (>= 256 routes per expert)
    MoeConfig(name="mfma_dma_shared", T=700, H=256, I=192, E=4, k=2, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=128, seed_index=30),
    MoeConfig(name="mfma_dma_gelu_bias", T=1100, H=128, I=320, E=2, k=1, act=ACT_GELU_TANH,
              weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, bias=BIAS_ZIPF,
              seed_index=31),
    # direct-to-LDS tiles with fewer routes per expert than a tile holds (the
    # weight operand three K-steps deep); K walks of 1 to 4 steps
    MoeConfig(name="mfma_dma_deep_shared", T=800, H=256, I=192, E=8, k=2, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=67),
    MoeConfig(name="mfma_dma_deep_short", T=900, H=128, I=64, E=8, k=2, act=ACT_GELU_TANH,
              weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, bias=BIAS_ZIPF,
              seed_index=68),
    # longer K walk (20 steps of 64) and 41 logit columns: ragged router tile
    MoeConfig(name="mfma_router_long_k", T=333, H=1280, I=64, E=40, k=3, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, bias=BIAS_ZIPF, shared=True, Is=64,
              seed_index=64),
    MoeConfig(name="mfma_t33", T=33, H=128, I=64, E=8, k=2, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=14),
    # 17 route tiles (16 experts + the shared one) in a grid sized for 19:
    # every XCD's share of tiles must still run (the grid is padded to a
    # multiple of 8 columns)
    MoeConfig(name="mfma_grid_tail", T=40, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=502),
    MoeConfig(name="mfma_dense_e1", T=40, H=128, I=64, E=1, k=1, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=15),
    # rows long enough that the router splits K in two ranges (partial
    # logits added by the top-k), shared gate column included
    MoeConfig(name="mfma_router_split", T=300, H=1024, I=64, E=16, k=4, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=505),
    # GEMV path
    MoeConfig(name="gemv_bf16x_shared", T=8, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=16),
    MoeConfig(name="gemv_f32_gelu_k_eq_e", T=16, H=128, I=96, E=8, k=8, act=ACT_GELU_TANH,
              seed_index=17),
    MoeConfig(name="gemv_u4_small", T=5, H=256, I=128, E=16, k=4, weight_format=WF_U4,
              seed_index=18),
    # 4-bit decode kernels: several staging passes per expert, bf16 x, one token, GELU
    MoeConfig(name="gemv_u4_passes", T=32, H=256, I=192, E=4, k=2, weight_format=WF_U4,
              seed_index=32),
    MoeConfig(name="gemv_u4_bf16x_gelu", T=9, H=512, I=64, E=8, k=3, act=ACT_GELU_TANH,
              weight_format=WF_U4, act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=33),
    MoeConfig(name="gemv_u4_t1", T=1, H=1024, I=320, E=16, k=4, weight_format=WF_U4,
              seed_index=34),
    MoeConfig(name="gemv_u4_many_routes", T=70, H=128, I=64, E=4, k=2, weight_format=WF_U4,
              seed_index=19),
    # rows long enough that only 3 routes fit a workgroup's LDS (3 per
    # work-list entry), and a group count (3) below one MFMA block row
    MoeConfig(name="gemv_u4_three_slots", T=6, H=9216, I=96, E=4, k=2, weight_format=WF_U4,
              seed_index=503),
    # one token, bf16 weights (gate/up activations straight from x), shared expert
    MoeConfig(name="gemv_bf16_shared_t1", T=1, H=1024, I=320, E=16, k=4, weight_format=WF_BF16,
              router_dtype=DT_BF16, shared=True, Is=192, seed_index=35),
    MoeConfig(name="gemv_bf16x_gelu_t1", T=1, H=512, I=256, E=64, k=8, act=ACT_GELU_TANH,
              weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=36),
    # one token ranked inside the gate/up kernel: experts past 128 (four
    # logits a lane, the last 64-expert block ragged), f32 weights, and 1, 2
    # or 4 features a wave
    MoeConfig(name="gemv_f32_t1_e256", T=1, H=192, I=96, E=256, k=8, seed_index=69),
    MoeConfig(name="gemv_bf16_t1_e129", T=1, H=2304, I=96, E=129, k=6, weight_format=WF_BF16,
              router_dtype=DT_BF16, shared=True, Is=32, seed_index=70),
    MoeConfig(name="gemv_bf16_t1_h4096", T=1, H=4096, I=32, E=8, k=2, act=ACT_GELU_TANH,
              weight_format=WF_BF16, seed_index=71),
    # one token: every expert selected (k = E), a single expert, and one
    # expert alone in the second 64-lane block of the ranking
    MoeConfig(name="gemv_f32_t1_k_eq_e", T=1, H=128, I=64, E=8, k=8, seed_index=81),
    MoeConfig(name="gemv_bf16_t1_dense_e1", T=1, H=128, I=64, E=1, k=1, weight_format=WF_BF16,
              router_dtype=DT_BF16, shared=True, Is=64, seed_index=82),
    MoeConfig(name="gemv_f32_t1_e65", T=1, H=96, I=32, E=65, k=3, seed_index=83),
    MoeConfig(name="gemv_f32_dense_e1", T=3, H=64, I=32, E=1, k=1, seed_index=20),
    MoeConfig(name="gemv_f32_k32", T=2, H=64, I=32, E=256, k=32, seed_index=21),
    MoeConfig(name="gemv_bf16_f32x_t32", T=32, H=2816, I=704, E=128, k=8, act=ACT_GELU_TANH,
              weight_format=WF_BF16, router_dtype=DT_BF16, seed_index=22),
    # few-token router launch: 64 and 200 experts (one and four logits a
    # lane in the per-token ranking)
    MoeConfig(name="gemv_route_rows_e64", T=32, H=128, I=64, E=64, k=6, seed_index=28),
    MoeConfig(name="gemv_route_rows_e200", T=20, H=64, I=32, E=200, k=5, weight_format=WF_BF16,
              router_dtype=DT_BF16, seed_index=29),
    # few-token router tiles: one, two and four token groups (the last ones
    # partly or wholly past T), one, two and four K slices, a ragged last
    # column block (shared gate column included), a router bias, 257 logit
    # columns (three quads a thread when the slices are added), three
    # logits a lane in the ranking
    MoeConfig(name="route_t8_bias_shared", T=8, H=8192, I=64, E=8, k=2, weight_format=WF_BF16,
              router_dtype=DT_BF16, bias=BIAS_ZIPF, shared=True, Is=64, seed_index=510),
    MoeConfig(name="route_t17_e41_shared", T=17, H=1024, I=64, E=41, k=5, act_dtype=DT_BF16,
              shared=True, Is=32, seed_index=511),
    MoeConfig(name="route_t32_e256_shared", T=32, H=512, I=32, E=256, k=8, weight_format=WF_BF16,
              router_dtype=DT_BF16, shared=True, Is=32, seed_index=512),
    MoeConfig(name="route_t25_u4_e192", T=25, H=2048, I=64, E=192, k=6, weight_format=WF_U4,
              seed_index=513),
    MoeConfig(name="route_t16_two_slices", T=16, H=4096, I=32, E=12, k=3, router_dtype=DT_BF16,
              seed_index=514),
    MoeConfig(name="route_t32_four_slices", T=32, H=4096, I=32, E=16, k=4, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, bias=BIAS_ZIPF, seed_index=515),
    MoeConfig(name="gemv_bf16_large_t_fallback", T=100, H=96, I=64, E=8, k=2,
              weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=23),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_shape_parity(cfg):
    check_case(Case(cfg))


def test_unnormalised_routing_parity():
    cfg = MoeConfig(name="mfma_nonorm", T=200, H=128, I=64, E=16, k=4, weight_format=WF_BF16,
                    act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=24)
    check_case(Case(cfg, normalize=False))
    cfg2 = MoeConfig(name="gemv_nonorm", T=4, H=64, I=32, E=8, k=2, seed_index=25)
    check_case(Case(cfg2, normalize=False))


# sigmoid gating and a routing-weight scale on every routing kernel: the
# decode router (wave per token at T <= 4, rows or ranks above), the prefill
# top-k kernel, and the 4-bit decode path; both with and without
# renormalisation
ROUTING_VARIANTS = [
    (MoeConfig(name="sig_decode_t3", T=3, H=128, I=64, E=16, k=4, seed_index=38),
     dict(gating=1, normalize=True, scale=2.5)),
    (MoeConfig(name="sig_decode_t20_raw", T=20, H=128, I=64, E=64, k=6, weight_format=WF_BF16,
               router_dtype=DT_BF16, seed_index=39), dict(gating=1, normalize=False, scale=0.5)),
    (MoeConfig(name="sig_decode_t1_bf16", T=1, H=1024, I=320, E=32, k=8, weight_format=WF_BF16,
               router_dtype=DT_BF16, shared=True, Is=128, seed_index=40),
     dict(gating=1, normalize=True, scale=1.0)),
    (MoeConfig(name="sig_prefill_shared", T=200, H=128, I=64, E=16, k=4, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=41),
     dict(gating=1, normalize=True, scale=1.75)),
    (MoeConfig(name="sig_prefill_raw", T=150, H=128, I=96, E=8, k=3, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=42),
     dict(gating=1, normalize=False, scale=1.0)),
    (MoeConfig(name="softmax_scaled_u4", T=6, H=256, I=128, E=16, k=4, weight_format=WF_U4,
               seed_index=43), dict(gating=0, normalize=True, scale=2.0)),
    (MoeConfig(name="sig_u4_raw", T=2, H=256, I=64, E=8, k=2, weight_format=WF_U4,
               seed_index=44), dict(gating=1, normalize=False, scale=3.0)),
]


@pytest.mark.parametrize("cfg,opts", ROUTING_VARIANTS, ids=[c.name for c, _ in ROUTING_VARIANTS])
def test_routing_variant_parity(cfg, opts):
    check_case(Case(cfg, **opts))


# per-expert routing scale (U(0.5, 1.5) per expert) on every routing
# kernel: one token ranked in the gate/up kernel (f32 and bf16 weights,
# past 128 experts), the wave-per-token decode routing, rank counting, row
# selection, the 4-bit decode path, the prefill top-k (MFMA path) and the
# GEMV fallback; softmax and sigmoid, with and without renormalisation
EXPERT_SCALE = [
    (MoeConfig(name="escale_t1_f32", T=1, H=192, I=96, E=200, k=8, seed_index=400),
     dict(gating=0, normalize=True)),
    (MoeConfig(name="escale_t1_bf16_shared_raw", T=1, H=1024, I=320, E=64, k=6,
               weight_format=WF_BF16, router_dtype=DT_BF16, shared=True, Is=128,
               seed_index=401), dict(gating=0, normalize=False, scale=1.5)),
    (MoeConfig(name="escale_t1_sigmoid", T=1, H=512, I=128, E=128, k=8, act=ACT_GELU_TANH,
               weight_format=WF_BF16, router_dtype=DT_BF16, seed_index=402),
     dict(gating=1, normalize=True)),
    (MoeConfig(name="escale_t3", T=3, H=128, I=64, E=16, k=4, seed_index=403),
     dict(gating=0, normalize=True)),
    (MoeConfig(name="escale_t8_rank_sigmoid", T=8, H=128, I=64, E=64, k=6, weight_format=WF_BF16,
               router_dtype=DT_BF16, seed_index=404), dict(gating=1, normalize=True)),
    (MoeConfig(name="escale_t20_rows", T=20, H=128, I=64, E=96, k=5, seed_index=405),
     dict(gating=0, normalize=True, scale=0.5)),
    (MoeConfig(name="escale_t20_rows_raw", T=20, H=128, I=64, E=96, k=5, seed_index=406),
     dict(gating=0, normalize=False)),
    (MoeConfig(name="escale_u4", T=6, H=256, I=128, E=16, k=4, weight_format=WF_U4,
               seed_index=407), dict(gating=0, normalize=True)),
    (MoeConfig(name="escale_prefill_shared", T=300, H=256, I=128, E=16, k=4,
               weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True,
               Is=64, seed_index=408), dict(gating=0, normalize=True)),
    (MoeConfig(name="escale_prefill_sigmoid_raw", T=200, H=128, I=64, E=8, k=3,
               weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=409),
     dict(gating=1, normalize=False, scale=2.0)),
    (MoeConfig(name="escale_gemv_fallback", T=100, H=96, I=64, E=8, k=2, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=410),
     dict(gating=0, normalize=True)),
]


@pytest.mark.parametrize("cfg,opts", EXPERT_SCALE, ids=[c.name for c, _ in EXPERT_SCALE])
def test_expert_scale_parity(cfg, opts):
    check_case(Case(cfg, expert_scale=True, **opts))


# pre-FFN RMSNorm on every path: decode (wave-per-token and one-token
# kernels), 4-bit decode, the MFMA prefill path and the GEMV fallback
PRE_NORM = [
    (MoeConfig(name="norm_decode_t3", T=3, H=128, I=64, E=16, k=4, seed_index=45), 1e-5),
    (MoeConfig(name="norm_decode_t1_bf16", T=1, H=1024, I=320, E=32, k=8, weight_format=WF_BF16,
               router_dtype=DT_BF16, shared=True, Is=128, seed_index=46), 1e-6),
    (MoeConfig(name="norm_prefill_shared", T=300, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=192, seed_index=47), 1e-5),
    (MoeConfig(name="norm_u4_bf16x", T=9, H=512, I=64, E=8, k=3, weight_format=WF_U4,
               act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=48), 1e-5),
    (MoeConfig(name="norm_gemv_fallback", T=100, H=96, I=64, E=8, k=2, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=49), 1e-5),
]


@pytest.mark.parametrize("cfg,eps", PRE_NORM, ids=[c.name for c, _ in PRE_NORM])
def test_pre_norm_parity(cfg, eps):
    check_case(Case(cfg, norm_eps=eps))


# residual folded into the kernel that writes out, on every path; also in
# place (residual == out)
RESIDUAL = [
    MoeConfig(name="res_decode_t4", T=4, H=128, I=64, E=8, k=2, seed_index=50),
    MoeConfig(name="res_decode_t1_bf16", T=1, H=1024, I=320, E=16, k=4, weight_format=WF_BF16,
              router_dtype=DT_BF16, seed_index=51),
    MoeConfig(name="res_u4", T=5, H=256, I=128, E=16, k=4, weight_format=WF_U4, seed_index=52),
    MoeConfig(name="res_prefill_shared", T=300, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=53),
    MoeConfig(name="res_gemv_fallback", T=100, H=96, I=64, E=8, k=2, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=54),
]


@pytest.mark.parametrize("cfg", RESIDUAL, ids=[c.name for c in RESIDUAL])
def test_residual_parity(cfg):
    import mixture_experts_ffn_gemv_amd as M
    from moe_synth import residual_values
    case = Case(cfg)
    r_host = residual_values(cfg)
    r = torch.from_numpy(r_host).cuda()
    log(f"[gpu] residual forward {cfg.name}")
    out = M.moe_ffn_forward(case.desc, case.dev.x, case.weights, residual=r)
    buf = r.clone()
    M.moe_ffn_forward(case.desc, case.dev.x, case.weights, out=buf, residual=buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, out), "in-place residual differs"
    toks = list(range(cfg.T))
    ffn = case.oracle_outputs(toks)
    got = out.cpu().numpy()
    # the layer's part, against the layer alone, and the sum against the oracle's sum
    assert rel_err(got - r_host, ffn) <= TOL_BY_WF[cfg.weight_format]
    assert rel_err(got, case.oracle_outputs(toks, residual=r_host)) <= TOL_BY_WF[cfg.weight_format]


def test_repeat_runs_bit_identical():
    case = Case(SMALL[0])
    a = case.forward()
    b = case.forward()
    for u, v in zip(a, b):
        assert (u == v).all()
    case2 = Case(CONFIGS["decode_geglu_t1"])
    assert (case2.forward()[0] == case2.forward()[0]).all()


def test_u4_rows_beyond_lds_are_unsupported_and_enqueue_nothing():
    # an intermediate row of 34816 4-bit values does not fit one
    # workgroup's LDS as a staged row: the call is refused before any launch
    import mixture_experts_ffn_gemv_amd as M
    cfg = MoeConfig(name="u4_too_long", T=2, H=256, I=34816, E=2, k=1, weight_format=WF_U4,
                    seed_index=504)
    case = Case(cfg)
    out = torch.full((cfg.T, cfg.H), 7.0, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.moe_ffn_forward(case.desc, case.dev.x, case.weights, out=out)
    assert ei.value.status == M.MOE_UNSUPPORTED and "LDS" in str(ei.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_error_path_enqueues_nothing():
    import mixture_experts_ffn_gemv_amd as M
    case = Case(CONFIGS["tiny_f32"])
    out = torch.full((4, 64), 7.0, device="cuda")
    ws = M.alloc_workspace(case.desc, 4)
    bad = M.make_desc(hidden=64, intermediate=32, num_experts=8, top_k=9)
    lib = M.load()
    st = lib.moe_ffn_forward(ctypes.byref(bad), 4, case.dev.x.data_ptr(), ctypes.byref(case.weights),
                             out.data_ptr(), None, None, None, ws.data_ptr(), ws.numel(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == M.MOE_INVALID_ARGUMENT
    st = lib.moe_ffn_forward(ctypes.byref(case.desc), 4, case.dev.x.data_ptr(),
                             ctypes.byref(case.weights), out.data_ptr(), None, None, None,
                             ws.data_ptr(), 64, torch.cuda.current_stream().cuda_stream)
    assert st == M.MOE_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    # zero tokens: nothing written either
    st = lib.moe_ffn_forward(ctypes.byref(case.desc), 0, case.dev.x.data_ptr(),
                             ctypes.byref(case.weights), out.data_ptr(), None, None, None,
                             ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == M.MOE_OK
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_zero_and_identity_weights_on_gpu():
    import mixture_experts_ffn_gemv_amd as M
    cfg = MoeConfig(name="ident", T=48, H=128, I=128, E=4, k=2, weight_format=WF_BF16,
                    act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=26)
    case = Case(cfg)
    eye = torch.eye(128, dtype=torch.bfloat16, device="cuda")
    for t in (case.dev.gate, case.dev.up, case.dev.down):
        t.copy_(eye.expand_as(t))
    out = M.moe_ffn_forward(case.desc, case.dev.x, case.weights)
    x = case.dev.x.float()
    ref = torch.nn.functional.silu(x.double()) * x.double()
    # bf16 intermediates (h and y are rounded to bf16 on the MFMA path)
    assert rel_err(out.cpu().numpy(), ref.cpu().numpy()) <= 2e-2
    for t in (case.dev.gate, case.dev.up, case.dev.down):
        t.zero_()
    out = M.moe_ffn_forward(case.desc, case.dev.x, case.weights)
    assert (out == 0).all()


def test_workspace_reuse_across_calls_and_token_counts():
    """One workspace serves a sequence of decode calls with changing token
    counts (routing-only calls in between): every call matches the oracle
    and the leading counter bytes are back at zero afterwards."""
    import mixture_experts_ffn_gemv_amd as M
    cfg = MoeConfig(name="ws_reuse", T=32, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
                    router_dtype=DT_BF16, seed_index=27)
    case = Case(cfg)
    ref_ids, ref_w = case.oracle_routing()
    ref_out = case.oracle_outputs(list(range(cfg.T)))
    ws = M.alloc_workspace(case.desc, cfg.T)
    for it, T in enumerate([1, 32, 5, 1, 17, 32, 2, 1]):
        x = case.dev.x[:T]
        log(f"[gpu] ws_reuse call {it}: T={T}")
        out, ids, w = M.moe_ffn_forward(case.desc, x, case.weights, workspace=ws,
                                        return_routing=True)
        if it % 3 == 1:
            r = M.moe_route(case.desc, x, case.weights, workspace=ws)
            torch.cuda.synchronize()
            assert (r.ids.cpu().numpy() == ref_ids[:T]).all()
        torch.cuda.synchronize()
        assert (ids.cpu().numpy() == ref_ids[:T]).all(), f"call {it} (T={T}): ids differ"
        assert float(np.abs(w.cpu().numpy() - ref_w[:T]).max()) <= 1e-5
        assert rel_err(out.cpu().numpy(), ref_out[:T]) <= 2e-2
    assert int(ws[:M.WORKSPACE_ZERO_BYTES].count_nonzero()) == 0



@pytest.mark.parametrize("name", ["decode_geglu_t1", "decode_u4_t32", "prefill_shared_t4096"])
def test_graph_replay_matches_eager(name):
    """The launch configuration bench.py times: the forward captured in a HIP
    graph and replayed.  Several replays, with eager work and
    synchronisations between them; each must equal the eager result bit for
    bit (the routing ticket is reset by the kernels, not by a memset)."""
    import mixture_experts_ffn_gemv_amd as M
    case = Case(CONFIGS[name])
    T = CONFIGS[name].T
    ws = M.alloc_workspace(case.desc, T)
    out = torch.empty((T, CONFIGS[name].H), dtype=torch.float32, device="cuda")
    ref = M.moe_ffn_forward(case.desc, case.dev.x, case.weights, workspace=ws).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.moe_ffn_forward(case.desc, case.dev.x, case.weights, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_ffn_forward(case.desc, case.dev.x, case.weights, out=out, workspace=ws)
    for it in range(4):
        out.fill_(float("nan"))
        log(f"[gpu] graph replay {it} {name}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {it} differs from the eager result"
        # eager work on the same workspace between replays
        e = M.moe_ffn_forward(case.desc, case.dev.x, case.weights, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(e, ref)
    assert int(ws[:M.WORKSPACE_ZERO_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("T", [2, 1])
def test_max_hidden_decode(T):
    """hidden = 16384, the largest the decode kernels take (several K passes
    per lane), bf16 weights; two tokens (routes staged in LDS) and one token
    (ranked in the gate/up kernel, four K blocks a lane)."""
    cfg = MoeConfig(name=f"decode_h16384_t{T}", T=T, H=16384, I=256, E=8, k=2,
                    weight_format=WF_BF16, router_dtype=DT_BF16, seed_index=55)
    check_case(Case(cfg))


# Exact ties in the router logits: integer router rows that repeat (or are
# all zero) and integer activations make equal logits bit-identical on both
# sides, so the lower expert index must win every tie, on every routing
# kernel: one token ranked in the gate/up kernel (up to 128 and past 128
# experts), the wave-per-token decode routing (T <= 4), rank counting (T*E
# <= 1024), row selection, and the prefill top-k after the MFMA router.
TIE_CASES = [
    (MoeConfig(name="ties_t1_e128", T=1, H=256, I=64, E=128, k=8, act=ACT_GELU_TANH,
               weight_format=WF_BF16, seed_index=74), False),
    (MoeConfig(name="ties_t1_e200", T=1, H=192, I=64, E=200, k=6, seed_index=75), False),
    (MoeConfig(name="ties_t1_zero", T=1, H=128, I=64, E=48, k=8, weight_format=WF_BF16,
               router_dtype=DT_BF16, seed_index=76), True),
    (MoeConfig(name="ties_t3", T=3, H=128, I=64, E=16, k=4, seed_index=77), False),
    (MoeConfig(name="ties_t8_rank", T=8, H=128, I=64, E=64, k=6, weight_format=WF_BF16,
               router_dtype=DT_BF16, seed_index=78), False),
    (MoeConfig(name="ties_t20_rows_zero", T=20, H=64, I=32, E=96, k=5, seed_index=79), True),
    (MoeConfig(name="ties_prefill", T=300, H=128, I=64, E=16, k=4, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=80), False),
]


@pytest.mark.parametrize("cfg,zero_top", TIE_CASES, ids=[c.name for c, _ in TIE_CASES])
def test_tied_logits_lowest_index_wins(cfg, zero_top):
    from moe_synth import tied_router_inputs
    from oracle import moe_oracle as O
    case = Case(cfg)
    r, x = tied_router_inputs(cfg, zero_top)
    case.dev.router.copy_(torch.from_numpy(r).to(case.dev.router.dtype))
    case.dev.x.copy_(torch.from_numpy(x).to(case.dev.x.dtype))
    torch.cuda.synchronize()
    # the inputs do tie inside every token's top k + 1 (and the logits are integers)
    L = O.router_logits(x.astype(np.float64), r.astype(np.float64), None)
    assert (L == np.round(L)).all()
    top = -np.sort(-L, axis=1)[:, :cfg.k + 1]
    assert (np.diff(top, axis=1) == 0).any(axis=1).all()
    check_case(case)


def _one_token_sweep(n=16, seed=0x1E7):
    """A fixed, seeded list of one-token layers for the in-kernel ranking:
    expert counts 1..256, k up to min(E, 32), row lengths and dtypes mixed,
    with or without a shared expert, softmax or sigmoid gating, with or
    without renormalisation, and a weight scale."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 7, 31, 64, 65, 100, 128, 129, 191, 256]))
        k = int(rng.integers(1, min(E, 32) + 1))
        wf = int(rng.choice([WF_F32, WF_BF16]))
        shared = bool(rng.integers(0, 2))
        cfg = MoeConfig(name=f"sweep_t1_{i}_e{E}_k{k}", T=1, H=32 * int(rng.integers(2, 33)),
                        I=32 * int(rng.integers(1, 9)), E=E, k=k,
                        act=int(rng.choice([ACT_SILU, ACT_GELU_TANH])), weight_format=wf,
                        act_dtype=int(rng.choice([DT_F32, DT_BF16])),
                        router_dtype=int(rng.choice([DT_F32, DT_BF16])), shared=shared,
                        Is=32 * int(rng.integers(1, 5)) if shared else 0, seed_index=100 + i)
        route = dict(gating=int(rng.integers(0, 2)), normalize=bool(rng.integers(0, 2)),
                     scale=float(rng.choice([1.0, 2.5])))
        out.append((cfg, route))
    return out


SWEEP = _one_token_sweep()


@pytest.mark.parametrize("cfg,route", SWEEP, ids=[c.name for c, _ in SWEEP])
def test_one_token_sweep(cfg, route):
    check_case(Case(cfg, **route))


def _few_token_sweep(n=10, seed=0x5E7):
    """A fixed, seeded list of 2..32-token decode layers: router rows of 64
    to 5120 elements (one to four K slices, one, two or four token groups),
    4 to 200 experts, f32, bf16 and 4-bit weights."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([2, 3, 4, 5, 9, 17, 32]))
        E = int(rng.choice([4, 16, 40, 64, 128, 200]))
        k = int(rng.integers(1, min(E, 8) + 1))
        wf = int(rng.choice([WF_F32, WF_BF16, WF_U4]))
        shared = wf != WF_U4 and bool(rng.integers(0, 2))
        cfg = MoeConfig(name=f"sweep_t{T}_{i}_e{E}_k{k}", T=T, H=32 * int(rng.integers(2, 161)),
                        I=32 * int(rng.integers(1, 7)), E=E, k=k,
                        act=int(rng.choice([ACT_SILU, ACT_GELU_TANH])), weight_format=wf,
                        act_dtype=int(rng.choice([DT_F32, DT_BF16])),
                        router_dtype=int(rng.choice([DT_F32, DT_BF16])), shared=shared,
                        Is=32 * int(rng.integers(1, 5)) if shared else 0, seed_index=200 + i)
        out.append(cfg)
    return out


FEW = _few_token_sweep()


@pytest.mark.parametrize("cfg", FEW, ids=[c.name for c in FEW])
def test_few_token_sweep(cfg):
    check_case(Case(cfg))


def _prefill_sweep(n=8, seed=0x9F1):
    """A fixed, seeded list of bf16 prefill layers (33..1200 tokens) whose
    experts average fewer or more than the 96 routes a tile needs for the
    direct-to-LDS GEMM, ragged in every tile dimension, with or without a
    shared expert and a router bias."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([2, 4, 8, 16, 32]))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(33, 1201))
        shared = bool(rng.integers(0, 2))
        cfg = MoeConfig(name=f"sweep_prefill_{i}_t{T}_e{E}_k{k}", T=T,
                        H=64 * int(rng.integers(1, 9)), I=64 * int(rng.integers(1, 7)), E=E, k=k,
                        act=int(rng.choice([ACT_SILU, ACT_GELU_TANH])), weight_format=WF_BF16,
                        act_dtype=DT_BF16, router_dtype=DT_BF16, shared=shared,
                        Is=64 * int(rng.integers(1, 4)) if shared else 0,
                        bias=int(rng.choice([0, BIAS_ZIPF])), seed_index=300 + i)
        out.append(cfg)
    return out


PREFILL_SWEEP = _prefill_sweep()


@pytest.mark.parametrize("cfg", PREFILL_SWEEP, ids=[c.name for c in PREFILL_SWEEP])
def test_prefill_sweep(cfg):
    check_case(Case(cfg))
