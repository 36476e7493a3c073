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
    assert lib.moe_abi_version() == 5


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
    ("routed_scale", float("nan")), ("pre_norm", 2)])
def test_bad_descriptor_is_invalid_argument(lib, field, value):
    d = _desc()
    setattr(d, field, value)          # raw field: bypass make_desc's coercions
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(d), 1, ctypes.byref(n))
    assert st == M.MOE_INVALID_ARGUMENT
    assert lib.moe_last_error().decode() != ""


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
