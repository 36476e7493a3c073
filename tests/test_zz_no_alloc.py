"""moe_ffn_forward_noalloc (the library's static scratch instead of a
workspace) against moe_ffn_forward with a workspace: two calls in a row on
each path, the second with fewer tokens, both bit-identical to the
workspace entry point (same kernels), and both within the oracle's
tolerance."""
import ctypes

import numpy as np
import pytest

from moe_synth import MoeConfig, CONFIGS, WF_BF16, WF_U4, DT_BF16, ACT_GELU_TANH

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_ffn_gemv_amd as M
    M.load()


from parity_util import Case, log, rel_err, TOL  # noqa: E402

# (layer, first token count, second token count): the one-token decode, the
# routing workgroup's path (its ticket lives in the scratch), 4-bit weights
# and the MFMA prefill path
NOALLOC_CASES = [
    (CONFIGS["decode_geglu_t1"], 1, 1),
    (MoeConfig(name="noalloc_decode_bf16", T=32, H=1024, I=256, E=64, k=6, act=ACT_GELU_TANH,
               weight_format=WF_BF16, router_dtype=DT_BF16, shared=True, Is=128,
               seed_index=500), 32, 5),
    (MoeConfig(name="noalloc_u4", T=32, H=512, I=256, E=16, k=4, weight_format=WF_U4,
               seed_index=501), 32, 7),
    (MoeConfig(name="noalloc_prefill", T=300, H=256, I=128, E=16, k=4, weight_format=WF_BF16,
               act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=64, seed_index=502),
     300, 40),
]


@pytest.mark.parametrize("cfg,t1,t2", NOALLOC_CASES, ids=[c.name for c, _, _ in NOALLOC_CASES])
def test_noalloc_matches_workspace_entry_point(cfg, t1, t2):
    import mixture_experts_ffn_gemv_amd as M
    case = Case(cfg)
    ref_ids, ref_w = case.oracle_routing()
    for T in (t1, t2):
        x = case.dev.x[:T]
        log(f"[gpu] noalloc {cfg.name} T={T}")
        a = M.moe_ffn_forward(case.desc, x, case.weights, return_routing=True)
        b = M.moe_ffn_forward_noalloc(case.desc, x, case.weights, return_routing=True)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v), f"{cfg.name} T={T}: no-alloc result differs"
        assert (b[1].cpu().numpy() == ref_ids[:T]).all()
        assert float(np.abs(b[2].cpu().numpy() - ref_w[:T]).max()) <= 1e-5
        ref = case.oracle_outputs(list(range(T)))
        assert rel_err(b[0].cpu().numpy(), ref) <= TOL[cfg.weight_format]


def test_noalloc_rejects_oversize_and_enqueues_nothing():
    import mixture_experts_ffn_gemv_amd as M
    cfg = CONFIGS["prefill_shared_t4096"]
    case = Case(cfg)
    need = M.workspace_size(case.desc, cfg.T)
    assert need > M.NOALLOC_SCRATCH_BYTES
    out = torch.full((cfg.T, cfg.H), 7.0, device="cuda")
    lib = M.load()
    st = lib.moe_ffn_forward_noalloc(ctypes.byref(case.desc), cfg.T, case.dev.x.data_ptr(),
                                     ctypes.byref(case.weights), out.data_ptr(), None, None, None,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == M.MOE_UNSUPPORTED
    assert "scratch" in lib.moe_last_error().decode()
    torch.cuda.synchronize()
    assert (out == 7.0).all()
