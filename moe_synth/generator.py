"""Counter-based seeded generator for the synthetic MoE FFN inputs.

Every value is a pure function of (master seed, tensor id, element index),
so any slice of any tensor can be produced on its own, on the CPU (numpy)
or on a GPU (torch integer/float64 ops), without generating the rest.

Definition (all integer arithmetic modulo 2**64):

* ``mix(z)`` is the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31``.
* ``key(seed, tensor) = mix(seed * G + tensor)`` with ``G = 0x9E3779B97F4A7C15``.
* ``bits(i) = mix(key + (i + 1) * G)`` for element counter ``i``.
* ``uniform(i) = ((bits(i) >> 11) + 0.5) * 2**-53``, strictly inside (0, 1).
* ``normal(i) = sqrt(-2 ln uniform(2i)) * cos(2 pi uniform(2i + 1))``
  (Box-Muller, cosine branch), evaluated in float64.
* a 4-bit code is ``bits(i) >> 60``.

Rounding into storage types is fixed as well: float64 -> float32 by
round-to-nearest-even, then float32 -> bfloat16 or float16 by
round-to-nearest-even.  bfloat16 values are held as their uint16 bit
patterns on the host and as ``torch.bfloat16`` on a device.

This module holds only the input recipe (distributions, shapes, seeds);
none of the layer's arithmetic.  The pages give no dataset for this layer:
all inputs are synthetic, with the shapes and distributions of the
workloads in ``configs.py``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import (MoeConfig, WF_F32, WF_BF16, WF_U4, DT_F32, DT_BF16,
                      BIAS_NONE, BIAS_ZIPF)

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# tensor ids (stream selectors)
TID_X = 1
TID_ROUTER = 2
TID_GATE = 3
TID_UP = 4
TID_DOWN = 5
TID_SH_GATE_INP = 6
TID_SH_GATE = 7
TID_SH_UP = 8
TID_SH_DOWN = 9
TID_NORM = 10          # pre-FFN RMSNorm weight [H]
TID_RESIDUAL = 11      # residual rows [T, H]
TID_GRAD_W = 12        # backward inputs: routing weights, y, dout, gate_up, dh
TID_GRAD_Y = 13
TID_GRAD_DOUT = 14
TID_GRAD_GU = 15
TID_U4_CODES = 16      # + matrix index (0 gate, 1 up, 2 down)
TID_GRAD_DH = 24
TID_U4_SCALES = 32     # + matrix index
TID_TIES_ROUTER = 40   # integer router rows with exact ties
TID_TIES_X = 41
TID_EXPERT_SCALE = 42  # per-expert routing scale [E]
ATTEMPT_SHIFT = 20     # resampled x rows use TID_X + (attempt << 20)


def mix_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * MIX1) & MASK64
    z ^= z >> 27
    z = (z * MIX2) & MASK64
    z ^= z >> 31
    return z


def stream_key(seed: int, tensor_id: int) -> int:
    return mix_int(seed * GOLDEN + tensor_id)


# ---------------------------------------------------------------- numpy side
def _mix_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * np.uint64(MIX1)
        z = z ^ (z >> np.uint64(27))
        z = z * np.uint64(MIX2)
        z = z ^ (z >> np.uint64(31))
    return z


def bits_np(key: int, idx: np.ndarray) -> np.ndarray:
    idx = idx.astype(np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GOLDEN)
    return _mix_np(z)


def uniform_np(key: int, idx: np.ndarray) -> np.ndarray:
    b = bits_np(key, idx) >> np.uint64(11)
    return (b.astype(np.float64) + 0.5) * (2.0 ** -53)


def normal_np(key: int, start: int, count: int) -> np.ndarray:
    i = np.arange(start, start + count, dtype=np.uint64)
    u1 = uniform_np(key, i * np.uint64(2))
    u2 = uniform_np(key, i * np.uint64(2) + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def codes_np(key: int, start: int, count: int) -> np.ndarray:
    i = np.arange(start, start + count, dtype=np.uint64)
    return (bits_np(key, i) >> np.uint64(60)).astype(np.uint8)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit constant as signed int64."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(z, s: int):
    """Logical right shift of an int64 tensor holding uint64 bits."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix_torch(z):
    z = z ^ _lsr(z, 30)
    z = z * _s64(MIX1)
    z = z ^ _lsr(z, 27)
    z = z * _s64(MIX2)
    z = z ^ _lsr(z, 31)
    return z


def bits_torch(key: int, idx):
    z = (idx + 1) * _s64(GOLDEN) + _s64(key)
    return _mix_torch(z)


def uniform_torch(key: int, idx):
    torch = _torch()
    b = _lsr(bits_torch(key, idx), 11)
    return (b.to(torch.float64) + 0.5) * (2.0 ** -53)


def normal_torch(key: int, start: int, count: int, device):
    torch = _torch()
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    u1 = uniform_torch(key, i * 2)
    u2 = uniform_torch(key, i * 2 + 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)


def codes_torch(key: int, start: int, count: int, device):
    torch = _torch()
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    return _lsr(bits_torch(key, i), 60).to(torch.uint8)


# ---------------------------------------------------------- tensor recipes
def _normal_tensor(seed, tid, shape, std, dtype, backend, device=None,
                   chunk=1 << 26):
    """N(0, std^2) tensor of ``shape`` stored as f32 or bf16."""
    n = int(np.prod(shape))
    key = stream_key(seed, tid)
    if backend == "numpy":
        out = np.empty(n, dtype=np.uint16 if dtype == DT_BF16 else np.float32)
        for s in range(0, n, 1 << 24):      # bounded temporaries
            c = min(1 << 24, n - s)
            v = (normal_np(key, s, c) * std).astype(np.float32)
            out[s:s + c] = f32_to_bf16_bits(v) if dtype == DT_BF16 else v
        return out.reshape(shape)
    torch = _torch()
    tdt = torch.bfloat16 if dtype == DT_BF16 else torch.float32
    out = torch.empty(n, dtype=tdt, device=device)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        v = normal_torch(key, s, c, device) * std
        out[s:s + c] = v.to(torch.float32).to(tdt)
    return out.view(shape)


@dataclass
class U4Weights:
    """Affine 4-bit weights, group ``g`` along K: w = code * scale + min.

    codes  : uint8 [E, N, K/2]; element 2i is the low nibble of byte i,
             element 2i+1 the high nibble
    scales : float16 [E, N, K/g]   (uint16 bits on the host)
    mins   : float16 [E, N, K/g]
    """
    codes: object
    scales: object
    mins: object
    K: int
    group: int


def _u4_tensor(seed, mat, E, N, K, group, backend, device=None, chunk=1 << 26):
    ng = K // group
    n_codes = E * N * K
    n_groups = E * N * ng
    kc = stream_key(seed, TID_U4_CODES + mat)
    ks = stream_key(seed, TID_U4_SCALES + mat)
    if backend == "numpy":
        packed = np.empty((E, N, K // 2), dtype=np.uint8)
        for e in range(E):                  # one expert at a time: bounded temporaries
            c = codes_np(kc, e * N * K, N * K).reshape(N, K)
            packed[e] = c[:, 0::2] | (c[:, 1::2] << 4)
        u = uniform_np(ks, np.arange(n_groups, dtype=np.uint64))
        sc = (0.005 + 0.015 * u).astype(np.float32).astype(np.float16)
        mn = (sc * np.float16(-8.0)).astype(np.float16)
        return U4Weights(packed, sc.view(np.uint16).reshape(E, N, ng),
                         mn.view(np.uint16).reshape(E, N, ng), K, group)
    torch = _torch()
    packed = torch.empty(n_codes // 2, dtype=torch.uint8, device=device)
    for s in range(0, n_codes, chunk):
        c = min(chunk, n_codes - s)
        cc = codes_torch(kc, s, c, device)
        packed[s // 2:(s + c) // 2] = cc[0::2] | (cc[1::2] << 4)
    i = torch.arange(n_groups, dtype=torch.int64, device=device)
    u = uniform_torch(ks, i)
    sc = (0.005 + 0.015 * u).to(torch.float32).to(torch.float16)
    mn = sc * -8.0
    return U4Weights(packed.view(E, N, K // 2), sc.view(E, N, ng),
                     mn.view(E, N, ng), K, group)


def _weight(seed, tid, mat, cfg, E, N, K, std, backend, device):
    if cfg.weight_format == WF_U4:
        return _u4_tensor(seed, mat, E, N, K, cfg.group_size, backend, device)
    dt = DT_BF16 if cfg.weight_format == WF_BF16 else DT_F32
    return _normal_tensor(seed, tid, (E, N, K), std, dt, backend, device)


def router_bias_values(cfg: MoeConfig) -> Optional[np.ndarray]:
    """Per-expert router bias (float32), or None when the workload has none.

    The skewed workload uses b_e = -2 ln(e + 1): rank e+1 gets a logit
    offset of 2 ln(1/rank), so low expert ids are picked far more often.
    """
    if cfg.bias == BIAS_NONE:
        return None
    if cfg.bias == BIAS_ZIPF:
        e = np.arange(cfg.E, dtype=np.float64)
        return (-2.0 * np.log(e + 1.0)).astype(np.float32)
    raise ValueError(f"unknown bias recipe {cfg.bias}")


@dataclass
class MoeInputs:
    """One workload's inputs in storage format (numpy on the host, or torch
    tensors on a device).  Layouts are row-major, weights are [out, in]."""
    cfg: MoeConfig
    x: object                 # [T, H]  f32 or bf16
    router: object            # [E, H]  router dtype
    router_bias: object       # [E] f32 or None
    gate: object              # [E, I, H] f32/bf16, or U4Weights
    up: object                # [E, I, H]
    down: object              # [E, H, I]
    shared_gate_inp: object = None   # [H]      router dtype
    shared_gate: object = None       # [Is, H]  weight dtype (f32/bf16)
    shared_up: object = None         # [Is, H]
    shared_down: object = None       # [H, Is]
    backend: str = "numpy"


def norm_weight_values(cfg: MoeConfig) -> np.ndarray:
    """Pre-FFN RMSNorm weight [H] (float32), uniform in [0.5, 1.5)."""
    key = stream_key(cfg.seed, TID_NORM)
    u = uniform_np(key, np.arange(cfg.H, dtype=np.uint64))
    return (0.5 + u).astype(np.float32)


def expert_scale_values(cfg: MoeConfig) -> np.ndarray:
    """Per-expert routing scale [E] (float32), uniform in [0.5, 1.5)."""
    key = stream_key(cfg.seed, TID_EXPERT_SCALE)
    u = uniform_np(key, np.arange(cfg.E, dtype=np.uint64))
    return (0.5 + u).astype(np.float32)


def residual_values(cfg: MoeConfig) -> np.ndarray:
    """Residual rows [T, H] (float32), N(0, 1)."""
    key = stream_key(cfg.seed, TID_RESIDUAL)
    return normal_np(key, 0, cfg.T * cfg.H).astype(np.float32).reshape(cfg.T, cfg.H)


def grad_inputs(cfg: MoeConfig) -> dict:
    """Inputs of the two backward steps at the workload's shape (float32):
    w [T, k] uniform (0, 1); y [T, k, H], dout [T, H], dh [T*k, I] N(0, 1);
    gate_up [T*k, 2I] N(0, 2^2), wide enough to reach both activation tails."""
    T, k, H, I, s = cfg.T, cfg.k, cfg.H, cfg.I, cfg.seed
    def nrm(tid, shape, std):
        n = int(np.prod(shape))
        return (normal_np(stream_key(s, tid), 0, n) * std).astype(np.float32).reshape(shape)
    w = uniform_np(stream_key(s, TID_GRAD_W), np.arange(T * k, dtype=np.uint64))
    return {"w": w.astype(np.float32).reshape(T, k), "y": nrm(TID_GRAD_Y, (T, k, H), 1.0),
            "dout": nrm(TID_GRAD_DOUT, (T, H), 1.0),
            "gate_up": nrm(TID_GRAD_GU, (T * k, 2 * I), 2.0),
            "dh": nrm(TID_GRAD_DH, (T * k, I), 1.0)}


def tied_router_inputs(cfg: MoeConfig, zero_top: bool = False):
    """Router rows [E, H] and token rows [T, H] (float32) of small integers,
    so that every logit is an exact integer in f32, bf16 inputs and f64
    alike, and equal logits are exact ties.  Default: rows repeat with
    period max(E // 4, 1) (experts e and e + E//4 tie), entries in -2..2,
    x in -3..3.  zero_top: every third expert (e % 3 == 1) has an all-zero
    row, so the largest logit is 0 (reached as +0 or -0 by the sums) for
    E/3 experts, the others -1 or below (entries in -2..0 with a -1 first,
    x in 1..3)."""
    E, H, T = cfg.E, cfg.H, cfg.T
    def ints(tid, n, lo, hi):
        u = uniform_np(stream_key(cfg.seed, tid), np.arange(n, dtype=np.uint64))
        return (lo + np.floor(u * (hi - lo + 1))).astype(np.float32)
    if zero_top:
        r = ints(TID_TIES_ROUTER, E * H, -2, 0).reshape(E, H)
        r[:, 0] = -1.0
        r[np.arange(E) % 3 == 1] = 0.0
        x = ints(TID_TIES_X, T * H, 1, 3).reshape(T, H)
    else:
        D = max(E // 4, 1)
        base = ints(TID_TIES_ROUTER, D * H, -2, 2).reshape(D, H)
        r = base[np.arange(E) % D]
        x = ints(TID_TIES_X, T * H, -3, 3).reshape(T, H)
    return r, x


def generate(cfg: MoeConfig, backend: str = "numpy", device=None) -> MoeInputs:
    """Generate every input of ``cfg`` (seed 0x5EED0000 + seed_index)."""
    s = cfg.seed
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    x = _normal_tensor(s, TID_X, (T, H), 1.0, cfg.act_dtype, backend, device)
    router = _normal_tensor(s, TID_ROUTER, (E, H), 1.0 / math.sqrt(H),
                            cfg.router_dtype, backend, device)
    b = router_bias_values(cfg)
    if b is not None and backend != "numpy":
        b = _torch().from_numpy(b).to(device)
    gate = _weight(s, TID_GATE, 0, cfg, E, I, H, 1.0 / math.sqrt(H), backend, device)
    up = _weight(s, TID_UP, 1, cfg, E, I, H, 1.0 / math.sqrt(H), backend, device)
    down = _weight(s, TID_DOWN, 2, cfg, E, H, I, 1.0 / math.sqrt(I), backend, device)
    inp = MoeInputs(cfg, x, router, b, gate, up, down, backend=backend)
    if cfg.shared:
        if cfg.weight_format == WF_U4:
            raise ValueError("shared expert with 4-bit weights is not a workload here")
        wdt = DT_BF16 if cfg.weight_format == WF_BF16 else DT_F32
        Is = cfg.Is
        inp.shared_gate_inp = _normal_tensor(s, TID_SH_GATE_INP, (H,), 1.0 / math.sqrt(H),
                                             cfg.router_dtype, backend, device)
        inp.shared_gate = _normal_tensor(s, TID_SH_GATE, (Is, H), 1.0 / math.sqrt(H),
                                         wdt, backend, device)
        inp.shared_up = _normal_tensor(s, TID_SH_UP, (Is, H), 1.0 / math.sqrt(H),
                                       wdt, backend, device)
        inp.shared_down = _normal_tensor(s, TID_SH_DOWN, (H, Is), 1.0 / math.sqrt(Is),
                                         wdt, backend, device)
    return inp


def x_rows(cfg: MoeConfig, rows, attempt: int, backend="numpy", device=None):
    """Fresh x rows (token ids ``rows``) drawn from the stream of ``attempt``.

    Used to redraw tokens whose router logits fall too close together; the
    caller decides which rows to redraw.
    """
    rows = list(rows)
    tid = TID_X + (attempt << ATTEMPT_SHIFT)
    key = stream_key(cfg.seed, tid)
    H = cfg.H
    out = []
    for t in rows:
        if backend == "numpy":
            v = (normal_np(key, t * H, H)).astype(np.float32)
            out.append(f32_to_bf16_bits(v) if cfg.act_dtype == DT_BF16 else v)
        else:
            torch = _torch()
            v = normal_torch(key, t * H, H, device).to(torch.float32)
            out.append(v.to(torch.bfloat16) if cfg.act_dtype == DT_BF16 else v)
    if backend == "numpy":
        return np.stack(out) if out else np.zeros((0, H), dtype=np.float32)
    return _torch().stack(out)
