"""GPU parity of the two backward kernels (routing-weighted combine and
gated activation) against the float64 oracle on seeded inputs.

dy = w * dout is one rounded f32 product on both sides: bit-exact.  dw is a
sum over H (f32 on the GPU): max|GPU-CPU| / max|CPU| <= 1e-5.  The gated
activation backward uses the same f32 exponential as the forward kernels:
max|GPU-CPU| / max|CPU| <= 1e-5."""
import numpy as np
import pytest

from moe_synth import MoeConfig, grad_inputs, ACT_SILU, ACT_GELU_TANH

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_ffn_gemv_amd as M
    M.load()


from parity_util import log, rel_err  # noqa: E402
from oracle import moe_oracle as O    # noqa: E402

TOL = 1e-5
SHAPES = [
    # ragged: H and I not multiples of a workgroup's 1024 / 2048 elements
    MoeConfig(name="bwd_ragged", T=37, H=200, I=100, E=8, k=3, seed_index=60),
    MoeConfig(name="bwd_k1", T=5, H=4, I=4, E=4, k=1, seed_index=61),
    MoeConfig(name="bwd_k32", T=3, H=2048, I=512, E=64, k=32, seed_index=62),
    # the 4096-token prefill shape (sampled rows against the oracle)
    MoeConfig(name="bwd_prefill_t4096", T=4096, H=2048, I=512, E=256, k=8, seed_index=63),
]


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_weighted_sum_backward_parity(cfg):
    import mixture_experts_ffn_gemv_amd as M
    g = grad_inputs(cfg)
    w, y, dout = _dev(g["w"]), _dev(g["y"]), _dev(g["dout"])
    log(f"[gpu] weighted_sum_backward {cfg.name} T={cfg.T} k={cfg.k} H={cfg.H}")
    dy, dw = M.weighted_sum_backward(w, y, dout)
    dy_only, _ = M.weighted_sum_backward(w, y, dout, need_dw=False)
    _, dw_only = M.weighted_sum_backward(w, y, dout, need_dy=False)
    torch.cuda.synchronize()
    assert torch.equal(dy, dy_only) and torch.equal(dw, dw_only)
    toks = list(range(cfg.T)) if cfg.T <= 64 else [0, 1, 1000, 2047, 4095]
    rdy, rdw = O.weighted_sum_backward(g["w"][toks], g["y"][toks], g["dout"][toks])
    got_dy = dy.cpu().numpy()[toks]
    # one correctly rounded f32 product on both sides
    assert (got_dy == rdy.astype(np.float32)).all()
    err = rel_err(dw.cpu().numpy()[toks], rdw)
    log(f"[parity] {cfg.name}: dw rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("act", [ACT_SILU, ACT_GELU_TANH], ids=["silu", "gelu_tanh"])
@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_glu_backward_parity(cfg, act):
    import mixture_experts_ffn_gemv_amd as M
    g = grad_inputs(cfg)
    gu, dh = _dev(g["gate_up"]), _dev(g["dh"])
    log(f"[gpu] glu_backward {cfg.name} rows={cfg.T * cfg.k} I={cfg.I} act={act}")
    out = M.glu_backward(gu, dh, act)
    torch.cuda.synchronize()
    R = cfg.T * cfg.k
    rows = list(range(R)) if R <= 512 else [0, 7, 4096, R // 2 + 3, R - 1]
    ref = O.glu_backward(g["gate_up"][rows], g["dh"][rows], act)
    err = rel_err(out.cpu().numpy()[rows], ref)
    log(f"[parity] {cfg.name} act={act}: rel err {err:.3e}")
    assert err <= TOL


def test_backward_rejects_bad_arguments_before_launch():
    import ctypes
    import mixture_experts_ffn_gemv_amd as M
    lib = M.load()
    x = torch.zeros(64, device="cuda")
    p = x.data_ptr()
    assert lib.moe_weighted_sum_backward(2, 0, 8, p, p, p, p, p, None) == M.MOE_INVALID_ARGUMENT
    assert lib.moe_weighted_sum_backward(2, 2, 6, p, p, p, p, p, None) == M.MOE_UNSUPPORTED
    assert lib.moe_weighted_sum_backward(2, 2, 8, p, p, p + 4, p, p, None) == M.MOE_UNSUPPORTED
    assert lib.moe_glu_backward(2, 8, 7, p, p, p, None) == M.MOE_INVALID_ARGUMENT
    assert lib.moe_glu_backward(2, 6, 0, p, p, p, None) == M.MOE_UNSUPPORTED
    assert lib.moe_glu_backward(0, 8, 0, None, None, None, None) == M.MOE_OK
    torch.cuda.synchronize()
    assert (x == 0).all()
