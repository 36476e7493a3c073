"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe_ffn.h declares, and rejects bad arguments on the host before
any HIP call."""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_gemv_amd as M
from moe_synth import CONFIGS
from moe_synth.device import desc_kwargs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe_ffn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from mixture_experts_ffn_gemv_amd.build import build
        build()
    return M.load()


def test_header_declares_the_bound_functions():
    assert _declared_functions() == sorted(M.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.moe_abi_version() == 8


def _desc(name="decode_geglu_t1", **over):
    kw = desc_kwargs(CONFIGS[name])
    kw.update(over)
    return M.make_desc(**kw)


def test_workspace_size_grows_affinely(lib):
    d = _desc("prefill_shared_t4096")
    sizes = [M.workspace_size(d, t) for t in (33, 1057, 2081, 3105)]
    # equal token steps (multiples of the tile and block sizes) give equal increments
    steps = [b - a for a, b in zip(sizes, sizes[1:])]
    assert max(steps) - min(steps) <= 4 * 256
    assert M.workspace_size(d, 0) > 0
    dd = _desc("decode_geglu_t1")
    assert M.workspace_size(dd, 1) < M.workspace_size(dd, 2) < M.workspace_size(dd, 32)


@pytest.mark.parametrize("field,value", [
    ("hidden", 0), ("intermediate", -32), ("num_experts", 0), ("num_experts", 257),
    ("top_k", 0), ("top_k", 129), ("activation", 5), ("weight_format", 7), ("act_dtype", 3),
    ("normalize_topk", 2), ("gating", 2), ("gating", -1), ("routed_scale", float("inf")),
    ("routed_scale", float("nan")), ("pre_norm", 2), ("out_dtype", 2), ("out_dtype", -1)])
def test_bad_descriptor_is_invalid_argument(lib, field, value):
    d = _desc()
    setattr(d, field, value)          # raw field: bypass make_desc's coercions
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n))
    assert st == M.MOE_INVALID_ARGUMENT
    assert lib.moe_last_error().decode() != ""


def test_bf16_output_unsupported(lib):
    d = _desc()
    d.out_dtype = M.DT_BF16
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == M.MOE_UNSUPPORTED
    assert "out_dtype" in lib.moe_last_error().decode()


def test_top_k_above_32_rejected(lib):
    d = _desc("prefill_shared_t4096", top_k=33)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == M.MOE_INVALID_ARGUMENT


def test_unaligned_sizes_unsupported(lib):
    d = _desc(hidden=100)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == M.MOE_UNSUPPORTED


def test_forward_rejects_null_and_small_workspace_on_host(lib):
    d = _desc()
    w = M.Weights()
    st = lib.moe_ffn_forward(ctypes.byref(d), 1, None, ctypes.byref(w), None, None, None, None, None,
                             0, None)
    assert st == M.MOE_INVALID_ARGUMENT
    # fake, aligned "device" addresses: validation fails before anything is enqueued
    fake = 1 << 20
    w = M.make_weights(router=None)
    w.router, w.gate, w.up, w.down = fake, fake, fake, fake
    st = lib.moe_ffn_forward(ctypes.byref(d), 1, fake, ctypes.byref(w), fake, None, None, None, fake,
                             16, None)
    assert st == M.MOE_WORKSPACE_TOO_SMALL
    assert "workspace" in lib.moe_last_error().decode()
    st = lib.moe_ffn_forward(ctypes.byref(d), -1, fake, ctypes.byref(w), fake, None, None, None,
                             fake, 1 << 30, None)
    assert st == M.MOE_INVALID_ARGUMENT
    st = lib.moe_ffn_forward(ctypes.byref(d), 1, fake + 4, ctypes.byref(w), fake, None, None, None,
                             fake, 1 << 30, None)
    assert st == M.MOE_UNSUPPORTED            # misaligned x


def test_wide_rows_need_the_bf16_prefill_path(lib):
    """Rows longer than 16384 are supported only on the bf16 MFMA path
    (bf16 weights and activations, more than 32 tokens); elsewhere the call
    is refused before anything is enqueued."""
    fake = 1 << 20
    w = M.make_weights(router=None)
    w.router, w.gate, w.up, w.down = fake, fake, fake, fake
    for name, T in (("decode_geglu_t1", 1), ("decode_geglu_t1", 8), ("decode_u4_t32", 32)):
        d = _desc(name, hidden=16416)
        if name == "decode_u4_t32":
            w.gate_u4 = w.up_u4 = w.down_u4 = M.U4Matrix(fake, fake, fake)
        st = lib.moe_ffn_forward(ctypes.byref(d), T, fake, ctypes.byref(w), fake, None, None, None,
                                 fake, 1 << 40, None)
        assert st == M.MOE_UNSUPPORTED, name
        assert "16384" in lib.moe_last_error().decode()
    d = _desc("prefill_shared_t4096", hidden=16448)
    assert M.workspace_size(d, 4096) > 0     # the bf16 prefill path plans it


def test_zero_tokens_is_a_noop(lib):
    d = _desc()
    w = M.Weights()
    assert lib.moe_ffn_forward(ctypes.byref(d), 0, None, ctypes.byref(w), None, None, None, None,
                               None, 0, None) == M.MOE_OK


def test_u4_needs_group_32(lib):
    d = _desc("decode_u4_t32", group_size=64)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == M.MOE_UNSUPPORTED


def test_workspace_zero_bytes_matches_header():
    import re
    with open(os.path.join(ROOT, "include", "moe_ffn.h")) as fh:
        m = re.search(r"#define MOE_WORKSPACE_ZERO_BYTES (\d+)", fh.read())
    assert m and int(m.group(1)) == M.WORKSPACE_ZERO_BYTES
    d = M.make_desc(hidden=64, intermediate=32, num_experts=8, top_k=2)
    assert M.workspace_size(d, 1) >= M.WORKSPACE_ZERO_BYTES


def test_pre_norm_needs_positive_eps_and_weight(lib):
    n = ctypes.c_size_t(0)
    for eps in (0.0, -1e-5, float("inf")):
        d = _desc(norm_eps=eps)
        assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == M.MOE_INVALID_ARGUMENT
    d = _desc(norm_eps=1e-5)
    assert lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n)) == M.MOE_OK
    fake = 1 << 20
    w = M.make_weights(router=None)
    w.router, w.gate, w.up, w.down = fake, fake, fake, fake     # no norm_weight
    st = lib.moe_ffn_forward(ctypes.byref(d), 1, fake, ctypes.byref(w), fake, None, None, None,
                             fake, 1 << 30, None)
    assert st == M.MOE_INVALID_ARGUMENT and "norm_weight" in lib.moe_last_error().decode()


def _packed_sizes_from_definition(H, I, E, Is):
    """Block counts of the packed layout the header defines: gate/up tiles of
    128 features and down tiles of 256 outputs, K-steps of 64, 32 KB blocks."""
    blk = 256 * 64 * 2
    gu = lambda n: -(-n // 128) * (H // 64) * blk
    dn = lambda n: -(-H // 256) * (n // 64) * blk
    return E * gu(I), E * dn(I), gu(Is) if Is else 0, dn(Is) if Is else 0


@pytest.mark.parametrize("H,I,E,Is", [(2048, 512, 256, 512), (7168, 2048, 256, 2048),
                                      (192, 64, 3, 192), (320, 192, 5, 0)])
def test_packed_weight_bytes(lib, H, I, E, Is):
    d = M.make_desc(hidden=H, intermediate=I, num_experts=E, top_k=2, weight_format=M.WEIGHTS_BF16,
                    act_dtype=M.DT_BF16, router_dtype=M.DT_BF16, shared_intermediate=Is)
    got = M.packed_weight_bytes(d)
    assert got == _packed_sizes_from_definition(H, I, E, Is)
    if I % 128 == 0:   # whole tiles: the same bytes as the row-major matrices
        assert got[0] == E * 2 * I * H * 2 and got[1] == E * H * I * 2 * (-(-H // 256) * 256) // H


@pytest.mark.parametrize("over", [dict(weight_format=M.WEIGHTS_F32, act_dtype=M.DT_F32),
                                  dict(intermediate=96), dict(shared_intermediate=160)])
def test_packed_weights_unsupported(lib, over):
    kw = dict(hidden=256, intermediate=128, num_experts=4, top_k=2, weight_format=M.WEIGHTS_BF16,
              act_dtype=M.DT_BF16, router_dtype=M.DT_BF16)
    kw.update(over)
    d = M.make_desc(**kw)
    n = ctypes.c_size_t(0)
    assert lib.moe_packed_weight_bytes(ctypes.byref(d), ctypes.byref(n), None, None,
                                       None) == M.MOE_UNSUPPORTED
    w = M.make_weights(router=None)
    fake = 1 << 20
    assert lib.moe_pack_weights(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, fake,
                                None) == M.MOE_UNSUPPORTED


def test_pack_weights_rejects_null_and_misaligned_on_host(lib):
    d = _desc("prefill_shared_t4096")
    fake = 1 << 20
    w = M.make_weights(router=None)
    assert lib.moe_pack_weights(ctypes.byref(d), None, fake, fake, fake, fake,
                                None) == M.MOE_INVALID_ARGUMENT
    w.gate, w.up, w.down = fake, fake, fake          # shared expert's matrices missing
    assert lib.moe_pack_weights(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, fake,
                                None) == M.MOE_INVALID_ARGUMENT
    w.shared_gate, w.shared_up, w.shared_down = fake, fake, fake
    assert lib.moe_pack_weights(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, None,
                                None) == M.MOE_INVALID_ARGUMENT
    assert lib.moe_pack_weights(ctypes.byref(d), ctypes.byref(w), fake, fake + 8, fake, fake,
                                None) == M.MOE_UNSUPPORTED


def test_forward_rejects_unpaired_packed_weights_on_host(lib):
    d = _desc("prefill_shared_t4096")
    fake = 1 << 20
    w = M.make_weights(router=None)
    w.router, w.gate, w.up, w.down = fake, fake, fake, fake
    w.shared_gate_inp, w.shared_gate, w.shared_up, w.shared_down = fake, fake, fake, fake
    w.gate_up_packed = fake                          # routed without shared
    st = lib.moe_ffn_forward(ctypes.byref(d), 4096, fake, ctypes.byref(w), fake, None, None, None,
                             fake, 1 << 40, None)
    assert st == M.MOE_INVALID_ARGUMENT and "packed" in lib.moe_last_error().decode()
    w.shared_gate_up_packed = fake + 4               # misaligned
    st = lib.moe_ffn_forward(ctypes.byref(d), 4096, fake, ctypes.byref(w), fake, None, None, None,
                             fake, 1 << 40, None)
    assert st == M.MOE_UNSUPPORTED
    dd = _desc("decode_u4_t32")                      # no packed layout for 4-bit weights
    w2 = M.make_weights(router=None)
    w2.router, w2.down_packed = fake, fake
    for name in ("gate_u4", "up_u4", "down_u4"):
        setattr(w2, name, M.U4Matrix(fake, fake, fake))
    st = lib.moe_ffn_forward(ctypes.byref(dd), 1, fake, ctypes.byref(w2), fake, None, None, None,
                             fake, 1 << 40, None)
    assert st == M.MOE_UNSUPPORTED


def test_noalloc_rejects_calls_beyond_its_scratch_on_host(lib):
    # the 4096-token prefill needs far more than the static scratch: the
    # call is refused on the host, before any HIP call
    d = _desc("prefill_shared_t4096")
    assert M.workspace_size(d, 4096) > M.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    w = M.make_weights(router=None)
    w.router, w.gate, w.up, w.down = fake, fake, fake, fake
    w.shared_gate_inp, w.shared_gate, w.shared_up, w.shared_down = fake, fake, fake, fake
    st = lib.moe_ffn_forward_noalloc(ctypes.byref(d), 4096, fake, ctypes.byref(w), fake, None,
                                     None, None, None)
    assert st == M.MOE_UNSUPPORTED and "scratch" in lib.moe_last_error().decode()
    # the bad-argument checks of moe_ffn_forward apply as well
    st = lib.moe_ffn_forward_noalloc(ctypes.byref(d), 4, None, ctypes.byref(w), fake, None,
                                     None, None, None)
    assert st == M.MOE_INVALID_ARGUMENT
    st = lib.moe_ffn_forward_noalloc(ctypes.byref(d), 0, fake, ctypes.byref(w), fake, None,
                                     None, None, None)
    assert st == M.MOE_OK


def test_noalloc_scratch_bytes_matches_header():
    src = open(os.path.join(ROOT, "include", "moe_ffn.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == M.NOALLOC_SCRATCH_BYTES
