"""Packed expert weights (moe_pack_weights).  The packed bytes must follow
the layout include/moe_ffn.h defines, byte for byte, and a forward pass that
reads them must give the same bits as one that reads the row-major matrices
(the operand tiles the GEMMs multiply are the same), hence the same oracle
parity."""
import numpy as np
import pytest

from moe_synth import CONFIGS, MoeConfig, WF_BF16, DT_BF16, ACT_GELU_TANH, BIAS_ZIPF

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_ffn_gemv_amd as M
    M.load()


from parity_util import Case, check_case, log  # noqa: E402

import mixture_experts_ffn_gemv_amd as M  # noqa: E402


def _slots(A):
    """A[..., r, c, 8] (row r, 16-byte chunk c) -> chunk c stored at slot c ^ ((r >> 1) & 7)."""
    r = np.arange(256)[:, None]
    q = np.arange(8)[None, :]
    src = q ^ ((r >> 1) & 7)           # slot q holds chunk q ^ swz (the XOR is an involution)
    idx = np.broadcast_to(src[..., None], A.shape[-3:])
    return np.take_along_axis(A, np.broadcast_to(idx, A.shape), axis=-2)


def expected_gate_up(g, u):
    """g, u: [E, N, K] bf16 bits -> packed bytes (tiles of 128 features)."""
    E, N, K = g.shape
    nwt = -(-N // 128)
    G = np.zeros((E, nwt * 128, K), np.uint16)
    U = np.zeros_like(G)
    G[:, :N], U[:, :N] = g, u
    A = np.concatenate([G.reshape(E, nwt, 128, K), U.reshape(E, nwt, 128, K)], axis=2)
    A = A.reshape(E, nwt, 256, K // 64, 8, 8).transpose(0, 1, 3, 2, 4, 5)
    return np.ascontiguousarray(_slots(A)).view(np.uint8).reshape(-1)


def expected_down(d):
    """d: [E, H, N] bf16 bits -> packed bytes (tiles of 256 outputs, K = N)."""
    E, H, N = d.shape
    nwt = -(-H // 256)
    D = np.zeros((E, nwt * 256, N), np.uint16)
    D[:, :H] = d
    A = D.reshape(E, nwt, 256, N // 64, 8, 8).transpose(0, 1, 3, 2, 4, 5)
    return np.ascontiguousarray(_slots(A)).view(np.uint8).reshape(-1)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


LAYOUT = [
    # ragged tiles: 64 of 128 gate/up features, 192 of 256 down outputs, Is = 192
    MoeConfig(name="pack_ragged", T=4, H=192, I=64, E=3, k=2, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True, Is=192, seed_index=65),
    MoeConfig(name="pack_whole", T=4, H=512, I=256, E=2, k=1, weight_format=WF_BF16,
              act_dtype=DT_BF16, router_dtype=DT_BF16, seed_index=66),
]


@pytest.mark.parametrize("cfg", LAYOUT, ids=lambda c: c.name)
def test_pack_layout_matches_definition(cfg):
    case = Case(cfg)
    dev = case.dev
    log(f"[gpu] moe_pack_weights {cfg.name}")
    bufs = M.pack_weights(case.desc, case.weights)
    torch.cuda.synchronize()
    exp = {"gate_up_packed": expected_gate_up(_bits(dev.gate), _bits(dev.up)),
           "down_packed": expected_down(_bits(dev.down))}
    if cfg.shared:
        exp["shared_gate_up_packed"] = expected_gate_up(_bits(dev.shared_gate)[None],
                                                        _bits(dev.shared_up)[None])
        exp["shared_down_packed"] = expected_down(_bits(dev.shared_down)[None])
    assert sorted(bufs) == sorted(exp)
    for name, want in exp.items():
        got = bufs[name].cpu().numpy()
        assert got.shape == want.shape, name
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{name}: {bad.size} bytes differ, first at {bad[:4]}"


# Workloads whose prefill GEMMs stream weight tiles (many routes per expert),
# and two whose paths do not use the packed arrays (fewer routes per expert;
# one-token decode), where giving them must change nothing
FORWARD = [
    "mfma_dma_shared", "mfma_dma_gelu_bias", "mfma_dma_deep_shared", "prefill_shared_t4096",
    "prefill_skew_t16384", "mfma_shared", "gemv_bf16_shared_t1",
]
SMALL = {
    "mfma_dma_shared": MoeConfig(name="mfma_dma_shared", T=700, H=256, I=192, E=4, k=2,
                                 weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16,
                                 shared=True, Is=128, seed_index=30),
    "mfma_dma_gelu_bias": MoeConfig(name="mfma_dma_gelu_bias", T=1100, H=128, I=320, E=2, k=1,
                                    act=ACT_GELU_TANH, weight_format=WF_BF16, act_dtype=DT_BF16,
                                    router_dtype=DT_BF16, bias=BIAS_ZIPF, seed_index=31),
    "mfma_dma_deep_shared": MoeConfig(name="mfma_dma_deep_shared", T=800, H=256, I=192, E=8, k=2,
                                      weight_format=WF_BF16, act_dtype=DT_BF16,
                                      router_dtype=DT_BF16, shared=True, Is=64, seed_index=67),
    "mfma_shared": MoeConfig(name="mfma_shared", T=300, H=256, I=128, E=16, k=4,
                             weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16,
                             shared=True, Is=192, seed_index=11),
    "gemv_bf16_shared_t1": MoeConfig(name="gemv_bf16_shared_t1", T=1, H=1024, I=320, E=16, k=4,
                                     weight_format=WF_BF16, router_dtype=DT_BF16, shared=True,
                                     Is=192, seed_index=35),
}


@pytest.mark.parametrize("name", FORWARD)
def test_packed_forward_is_bit_identical(name):
    cfg = SMALL.get(name) or CONFIGS[name]
    case = Case(cfg)
    out0, ids0, w0 = case.forward()
    bufs = M.pack_weights(case.desc, case.weights)
    out1, ids1, w1 = case.forward()
    assert (ids0 == ids1).all() and (w0 == w1).all()
    diff = np.flatnonzero(out0.view(np.uint32) != out1.view(np.uint32))
    assert diff.size == 0, f"{name}: {diff.size} outputs differ with packed weights"
    if name in SMALL:
        check_case(case)                     # and so the oracle parity, read from packed
    del bufs


def test_packed_arrays_are_the_ones_read():
    """Zeroing the packed down weights zeroes the routed experts' output."""
    case = Case(SMALL["mfma_dma_gelu_bias"])
    out0, _, _ = case.forward()
    assert np.abs(out0).max() > 0
    bufs = M.pack_weights(case.desc, case.weights)
    bufs["down_packed"].zero_()
    out1, _, _ = case.forward()
    assert (out1 == 0).all()
    case.weights.gate_up_packed = None       # unpacked again: the row-major result
    case.weights.down_packed = None
    out2, _, _ = case.forward()
    assert (out2.view(np.uint32) == out0.view(np.uint32)).all()
