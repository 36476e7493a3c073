"""Python binding of the gfx950 MoE FFN library (libmoe_ffn.so).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels; torch supplies device memory (tensors, workspace) and the
current stream.  The functions mirror the C ABI in include/moe_ffn.h:

    workspace_size(desc, T)
    moe_route(desc, x, weights, ...)      -> ids, w, counts, offsets, perm
    moe_ffn_forward(desc, x, weights, ...) -> out [T, H] f32 (+ ids, w)

Loading fails loudly when the library has not been built (see build.py);
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_ffn.so")

MOE_OK = 0
MOE_INVALID_ARGUMENT = 1
MOE_UNSUPPORTED = 2
MOE_WORKSPACE_TOO_SMALL = 3
MOE_HIP_ERROR = 4
WORKSPACE_ZERO_BYTES = 256   # MOE_WORKSPACE_ZERO_BYTES: leading bytes zeroed before first use

WEIGHTS_F32, WEIGHTS_BF16, WEIGHTS_U4_G32 = 0, 1, 2
ACT_SILU, ACT_GELU_TANH = 0, 1
GATING_SOFTMAX, GATING_SIGMOID = 0, 1
DT_F32, DT_BF16 = 0, 1

EXPORTED_SYMBOLS = ("moe_abi_version", "moe_last_error", "moe_workspace_size", "moe_route",
                    "moe_ffn_forward", "moe_ffn_forward_noalloc", "moe_weighted_sum_backward",
                    "moe_glu_backward",
                    "moe_packed_weight_bytes", "moe_pack_weights",
                    "moe_timing_enable", "moe_timing_read", "moe_timing_reset")


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe status {status}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "intermediate", "num_experts", "top_k", "activation", "weight_format",
        "act_dtype", "router_dtype", "normalize_topk", "has_shared_expert",
        "shared_intermediate", "group_size", "gating")] + [
        ("routed_scale", ctypes.c_float), ("pre_norm", ctypes.c_int32),
        ("norm_eps", ctypes.c_float), ("out_dtype", ctypes.c_int32)]


class U4Matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("mins", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_u4", U4Matrix), ("up_u4", U4Matrix), ("down_u4", U4Matrix),
                ("shared_gate_inp", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p),
                ("shared_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p),
                ("norm_weight", ctypes.c_void_p),
                ("gate_up_packed", ctypes.c_void_p), ("down_packed", ctypes.c_void_p),
                ("shared_gate_up_packed", ctypes.c_void_p),
                ("shared_down_packed", ctypes.c_void_p), ("expert_scale", ctypes.c_void_p)]


_lib = None


def load(path: Optional[str] = None):
    """Load libmoe_ffn.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} not found: build it with `python -m mixture_experts_ffn_gemv_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.moe_abi_version.restype = i32
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_workspace_size.argtypes = [ctypes.POINTER(Desc), i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_workspace_size.restype = i32
    lib.moe_route.argtypes = [ctypes.POINTER(Desc), i64, vp, ctypes.POINTER(Weights), vp, vp, vp,
                              vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_route.restype = i32
    lib.moe_ffn_forward.argtypes = [ctypes.POINTER(Desc), i64, vp, ctypes.POINTER(Weights), vp, vp,
                                    vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_ffn_forward.restype = i32
    lib.moe_ffn_forward_noalloc.argtypes = [ctypes.POINTER(Desc), i64, vp, ctypes.POINTER(Weights),
                                            vp, vp, vp, vp, vp]
    lib.moe_ffn_forward_noalloc.restype = i32
    lib.moe_weighted_sum_backward.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.moe_weighted_sum_backward.restype = i32
    lib.moe_glu_backward.argtypes = [i64, i32, i32, vp, vp, vp, vp]
    lib.moe_glu_backward.restype = i32
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.moe_packed_weight_bytes.argtypes = [ctypes.POINTER(Desc), szp, szp, szp, szp]
    lib.moe_packed_weight_bytes.restype = i32
    lib.moe_pack_weights.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Weights), vp, vp, vp,
                                     vp, vp]
    lib.moe_pack_weights.restype = i32
    lib.moe_timing_enable.argtypes = [i32]
    lib.moe_timing_enable.restype = i32
    lib.moe_timing_read.argtypes = [ctypes.c_char_p, i32, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_double), i32]
    lib.moe_timing_read.restype = i32
    lib.moe_timing_reset.restype = i32
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode())


def make_desc(hidden, intermediate, num_experts, top_k, activation=ACT_SILU,
              weight_format=WEIGHTS_BF16, act_dtype=DT_F32, router_dtype=DT_F32,
              normalize_topk=True, shared_intermediate=0, group_size=32,
              gating=GATING_SOFTMAX, routed_scale=1.0, norm_eps=None, out_dtype=DT_F32) -> Desc:
    """``norm_eps`` (a float) turns on the pre-FFN RMSNorm (weights need norm_weight);
    ``out_dtype``: the output's dtype (only DT_F32 is supported)."""
    return Desc(hidden, intermediate, num_experts, top_k, activation, weight_format, act_dtype,
                router_dtype, int(bool(normalize_topk)), int(shared_intermediate > 0),
                shared_intermediate, group_size, gating, routed_scale,
                int(norm_eps is not None), 0.0 if norm_eps is None else norm_eps, out_dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_weights(router, gate=None, up=None, down=None, router_bias=None, shared_gate_inp=None,
                 shared_gate=None, shared_up=None, shared_down=None, u4=None,
                 norm_weight=None, expert_scale=None) -> Weights:
    """Device tensors -> moe_weights.  ``u4`` = dict(gate=(codes, scales, mins), up=..., down=...);
    ``expert_scale``: [E] float32 per-expert routing scale, or None."""
    w = Weights()
    w.router, w.router_bias = _ptr(router), _ptr(router_bias)
    w.gate, w.up, w.down = _ptr(gate), _ptr(up), _ptr(down)
    if u4 is not None:
        for name in ("gate", "up", "down"):
            c, s, m = u4[name]
            setattr(w, name + "_u4", U4Matrix(_ptr(c), _ptr(s), _ptr(m)))
    w.shared_gate_inp, w.shared_gate = _ptr(shared_gate_inp), _ptr(shared_gate)
    w.shared_up, w.shared_down = _ptr(shared_up), _ptr(shared_down)
    w.norm_weight = _ptr(norm_weight)
    w.expert_scale = _ptr(expert_scale)
    return w


def workspace_size(desc: Desc, num_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(desc), num_tokens, ctypes.byref(n)))
    return n.value


PACKED_FIELDS = ("gate_up_packed", "down_packed", "shared_gate_up_packed", "shared_down_packed")


def packed_weight_bytes(desc: Desc) -> tuple:
    """Sizes of (gate_up, down, shared_gate_up, shared_down) packed arrays."""
    n = [ctypes.c_size_t(0) for _ in range(4)]
    _check(load().moe_packed_weight_bytes(ctypes.byref(desc), *[ctypes.byref(v) for v in n]))
    return tuple(v.value for v in n)


def pack_weights(desc: Desc, weights: Weights, device="cuda", stream=None) -> dict:
    """Packs the bf16 expert weights of ``weights`` into new device arrays and
    points ``weights``' packed fields at them; returns the arrays (keep them
    alive while ``weights`` is in use)."""
    import torch
    sizes = packed_weight_bytes(desc)
    bufs = {n: torch.empty(sz, dtype=torch.uint8, device=device)
            for n, sz in zip(PACKED_FIELDS, sizes) if sz}
    ptrs = [_ptr(bufs.get(n)) for n in PACKED_FIELDS]
    _check(load().moe_pack_weights(ctypes.byref(desc), ctypes.byref(weights), *ptrs,
                                   _stream(stream)))
    for n, q in zip(PACKED_FIELDS, ptrs):
        setattr(weights, n, q)
    return bufs


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def alloc_workspace(desc: Desc, num_tokens: int, device="cuda"):
    import torch
    # zero-filled: the leading counter bytes must start at zero (calls keep them so)
    return torch.zeros(max(workspace_size(desc, num_tokens), WORKSPACE_ZERO_BYTES), dtype=torch.uint8, device=device)


@dataclass
class RouteResult:
    ids: object
    weights: object
    counts: object
    offsets: object
    perm: object


def moe_route(desc: Desc, x, weights: Weights, workspace=None, stream=None) -> RouteResult:
    import torch
    T = x.shape[0]
    k, E = desc.top_k, desc.num_experts
    dev = x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = workspace if workspace is not None else alloc_workspace(desc, T, dev)
    _check(load().moe_route(ctypes.byref(desc), T, x.data_ptr(), ctypes.byref(weights),
                            ids.data_ptr(), w.data_ptr(), counts.data_ptr(), offsets.data_ptr(),
                            perm.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    return RouteResult(ids, w, counts, offsets, perm)


def moe_ffn_forward(desc: Desc, x, weights: Weights, out=None, workspace=None, stream=None,
                    return_routing: bool = False, residual=None):
    """out = layer(x) (+ residual, a float32 [T, H] tensor, which may be ``out``)."""
    import torch
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, desc.hidden), dtype=torch.float32, device=dev)
    ids = w = None
    if return_routing:
        ids = torch.empty((T, desc.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, desc.top_k), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else alloc_workspace(desc, T, dev)
    _check(load().moe_ffn_forward(ctypes.byref(desc), T, x.data_ptr(), ctypes.byref(weights),
                                  out.data_ptr(), _ptr(residual), _ptr(ids), _ptr(w),
                                  ws.data_ptr(), ws.numel(), _stream(stream)))
    return (out, ids, w) if return_routing else out


NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def moe_ffn_forward_noalloc(desc: Desc, x, weights: Weights, out=None, stream=None,
                            return_routing: bool = False, residual=None):
    """moe_ffn_forward on the library's static scratch (no workspace)."""
    import torch
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, desc.hidden), dtype=torch.float32, device=dev)
    ids = w = None
    if return_routing:
        ids = torch.empty((T, desc.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, desc.top_k), dtype=torch.float32, device=dev)
    _check(load().moe_ffn_forward_noalloc(ctypes.byref(desc), T, x.data_ptr(),
                                          ctypes.byref(weights), out.data_ptr(), _ptr(residual),
                                          _ptr(ids), _ptr(w), _stream(stream)))
    return (out, ids, w) if return_routing else out


def weighted_sum_backward(w, y, dout, need_dy: bool = True, need_dw: bool = True, stream=None):
    """Gradients of out[t] = sum_j w[t,j] y[t,j] (float32 tensors w [T,k],
    y [T,k,H], dout [T,H]): returns (dy [T,k,H] or None, dw [T,k] or None)."""
    import torch
    T, k = w.shape
    H = dout.shape[1]
    dy = torch.empty((T, k, H), dtype=torch.float32, device=w.device) if need_dy else None
    dw = torch.empty((T, k), dtype=torch.float32, device=w.device) if need_dw else None
    _check(load().moe_weighted_sum_backward(T, k, H, w.data_ptr(), _ptr(y), dout.data_ptr(),
                                            _ptr(dy), _ptr(dw), _stream(stream)))
    return dy, dw


def glu_backward(gate_up, dh, activation=ACT_SILU, out=None, stream=None):
    """Gradients of h = act(g) * u for gate_up [R, 2I] (g | u) and dh [R, I]:
    returns d_gate_up [R, 2I] (dg | du), float32."""
    import torch
    R, I2 = gate_up.shape
    if out is None:
        out = torch.empty((R, I2), dtype=torch.float32, device=gate_up.device)
    _check(load().moe_glu_backward(R, I2 // 2, activation, gate_up.data_ptr(), dh.data_ptr(),
                                   out.data_ptr(), _stream(stream)))
    return out


def timing_enable(on: bool = True):
    _check(load().moe_timing_enable(1 if on else 0))


def timing_reset():
    _check(load().moe_timing_reset())


def timing_read(max_entries: int = 32):
    """{kernel name: (launches, total_ms)} accumulated since the last reset."""
    stride = 64
    names = ctypes.create_string_buffer(stride * max_entries)
    launches = (ctypes.c_int64 * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    n = load().moe_timing_read(names, stride, launches, ms, max_entries)
    if n < 0:
        raise MoeError(MOE_INVALID_ARGUMENT, "moe_timing_read failed")
    out = {}
    for i in range(n):
        nm = names.raw[i * stride:(i + 1) * stride].split(b"\0", 1)[0].decode()
        out[nm] = (launches[i], ms[i])
    return out
