"""CPU oracle for the mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP
library; the two meet only in the seeded inputs of ``moe_synth``.

It is a plain, slow, float64 implementation of the layer in the op order
that hf2q's qwen35/gpu_ffn.rs states in its module header ("MoE FFN op
order"):

1. router logits  l = x . Wr^T  (+ per-expert bias, as ferrox-models
   decoder.rs adds in gpt_oss_ffn before selection)
2. softmax over all experts (or a sigmoid per expert), top-k by score
   (stable sort, so the lower expert index wins a tie), optionally times a
   per-expert scale (mlx-native moe_gather_topk_weights_encode),
   renormalise the k selected scores to sum to one (hf2q
   softmax_topk_renorm_cpu), times a weight scale
3. for each selected expert e: g = Wg[e] x, u = Wu[e] x,
   h = act(g) * u, y = Wd[e] h; out += w * y, in slot order
4. shared expert (when present): s = sigmoid(x . w_sg),
   y_s = Wsd (silu(Wsg x) * Wsu x), out += s * y_s
5. out is returned as float64 (the library writes float32), plus an
   optional residual; the input may first go through the pre-FFN RMSNorm

plus the expert-grouping permutation (a stable counting sort of the flat
route ids by expert, as DS4Server qwen_mtplx.rs gather_sort obtains with an
argsort of the flat expert ids, and ferrox-models moe_ffn_batch builds by
bucketing tokens per expert in token order).

Activations: SiLU z/(1+e^-z) (hf2q silu_mul_cpu) and the tanh form of GELU
0.5 z (1 + tanh(0.7978845608 (z + 0.044715 z^3))) that mlx-native's
moe_dispatch.rs tests use as their float64 oracle (cpu_gelu).

Storage decoding is exact: f32 as is, bf16 by placing the 16 bits in the
top half of an f32, f16 by IEEE binary16, and 4-bit affine codes as
code * scale + min in float64.

Every function here is pinned by the not-gpu tests (closed forms, brute
force on tiny inputs, special cases that reduce to a dense FFN).  The full
outputs at the large workload shapes have no printed worked example on the
pages: beyond the invariants, parity at those shapes is unpinned.
"""
from __future__ import annotations

import numpy as np

SQRT_2_OVER_PI = 0.7978845608   # constant as printed for the tanh GELU
GELU_CUBIC = 0.044715

ACT_SILU = 0
ACT_GELU_TANH = 1


# ------------------------------------------------------------ storage decode
def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def u4_dequant(codes, scales_bits, mins_bits, K: int, group: int) -> np.ndarray:
    """Affine 4-bit rows: w[n, c] = code[n, c] * scale[n, c//g] + min[n, c//g].

    ``codes`` is uint8 [N, K/2] with element 2i in the low nibble of byte i
    and element 2i+1 in the high nibble; scale/min are f16 [N, K/g].  This is
    the affine (scale, bias) form that hf2q's dispatch_moe_id_routed passes
    to its quantized matmul, with the nibble order fixed here.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[0]
    q = np.empty((N, K), dtype=np.float64)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    s = np.repeat(f16_to_f64(scales_bits), group, axis=1)
    m = np.repeat(f16_to_f64(mins_bits), group, axis=1)
    return q * s + m


def decode_matrix(a, is_bf16: bool) -> np.ndarray:
    if is_bf16:
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- activations
def silu(z):
    """SiLU(z) = z / (1 + exp(-z))  (hf2q silu_mul_cpu)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    """tanh-approximate GELU (mlx-native moe_dispatch.rs, cpu_gelu oracle)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(SQRT_2_OVER_PI * (z + GELU_CUBIC * z * z * z)))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def activation(kind: int, z):
    if kind == ACT_SILU:
        return silu(z)
    if kind == ACT_GELU_TANH:
        return gelu_tanh(z)
    raise ValueError(f"unknown activation {kind}")


# -------------------------------------------------------------------- routing
def router_logits(x, Wr, bias=None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h] (+ b[e]); all float64.

    hf2q gpu_ffn.rs op order, step 1 (router projection, x . Wr^T).
    """
    l = np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def rms_norm(X, w, eps: float) -> np.ndarray:
    """Pre-FFN RMSNorm of token rows: x / sqrt(mean(x^2) + eps) * w.

    ferrox-models decoder.rs runs the MoE block on rms_norm(hidden,
    norm_weight, rms_norm_eps); the pages call it without printing its
    arithmetic, so this is the usual definition (mean over the hidden
    dimension, eps inside the square root, weight applied last).
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    ms = (X * X).mean(axis=1, keepdims=True)
    return X / np.sqrt(ms + float(eps)) * np.asarray(w, dtype=np.float64)[None, :]


def round_to_act(X, bf16: bool) -> np.ndarray:
    """Values as the layer stores its normalised input: float32, then (for
    bf16 activations) bfloat16, each by round-to-nearest-even."""
    f = np.asarray(X, dtype=np.float64).astype(np.float32)
    if not bf16:
        return f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    return bf16_to_f64(r.astype(np.uint16))


def softmax_row(l) -> np.ndarray:
    """Max-subtracted softmax over one token's logits (softmax_topk_renorm_cpu)."""
    l = np.asarray(l, dtype=np.float64)
    e = np.exp(l - l.max())
    return e / e.sum()


def topk_stable_desc(p, k: int) -> np.ndarray:
    """Indices of the k largest entries, in descending order of value.

    A stable sort over indices 0..E-1 keyed on -p keeps equal values in
    index order, so the lower expert index comes first among ties (the
    stable ``sort_by`` of softmax_topk_renorm_cpu).
    """
    p = np.asarray(p, dtype=np.float64)
    order = sorted(range(len(p)), key=lambda i: -p[i])   # Python's sort is stable
    return np.array(order[:k], dtype=np.int64)


GATING_SOFTMAX = 0
GATING_SIGMOID = 1


def gating_scores(l, gating: int = GATING_SOFTMAX) -> np.ndarray:
    """Routing scores of one token's logits.

    Softmax over all experts (hf2q softmax_topk_renorm_cpu), or one sigmoid
    per expert, the other gating function ferrox-models decoder.rs routes
    with (its dense-layer note: sigmoid scores, then renormalisation
    divides the selected score by the selected sum).
    """
    if gating == GATING_SOFTMAX:
        return softmax_row(l)
    if gating == GATING_SIGMOID:
        return sigmoid(l)
    raise ValueError(f"unknown gating {gating}")


def route(logits, k: int, normalize: bool = True, gating: int = GATING_SOFTMAX,
          scale: float = 1.0, expert_scale=None):
    """Scores -> top-k -> per-expert scale -> renormalise -> scale, per token.

    Returns (ids [T, k] int64, weights [T, k] float64); slot j holds the
    j-th largest score.  Selection looks at the scores only.  With
    ``expert_scale`` ([E]) each selected score is first multiplied by its
    expert's entry, and the renormalisation then runs over those scaled
    scores: the order of mlx-native moe_dispatch.rs
    moe_gather_topk_weights_encode (gather the top-k ids and weights, apply
    per_expert_scale, renormalise).  Without ``normalize`` the (scaled) raw
    scores of the winners are returned.  Every weight is then multiplied by
    ``scale`` (llama.cpp's w_scale, which ferrox-models names in
    gpt_oss_ffn; the pages give only the name and the value 1, so a plain
    factor on the weights is the reading taken).
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T = logits.shape[0]
    ids = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k), dtype=np.float64)
    es = None if expert_scale is None else np.asarray(expert_scale, dtype=np.float64)
    for t in range(T):
        p = gating_scores(logits[t], gating)
        sel = topk_stable_desc(p, k)
        ids[t] = sel
        ps = p[sel]
        if es is not None:
            ps = ps * es[sel]
        w[t] = (ps / ps.sum() if normalize else ps) * scale
    return ids, w


# ------------------------------------------------------------------ backward
# The two backward steps mlx-native's moe_dispatch.rs adds for training
# (moe_weighted_sum_seq and moe_swiglu_seq backward), as printed there.
def weighted_sum(w, y):
    """out[t, d] = sum_j w[t, j] y[t, j, d] (the routing-weighted combine)."""
    return np.einsum("tj,tjd->td", np.asarray(w, np.float64), np.asarray(y, np.float64))


def weighted_sum_backward(w, y, dout):
    """dy[t,j,d] = w[t,j] dout[t,d];  dw[t,j] = sum_d y[t,j,d] dout[t,d]."""
    w = np.asarray(w, np.float64)
    y = np.asarray(y, np.float64)
    dout = np.asarray(dout, np.float64)
    return w[:, :, None] * dout[:, None, :], np.einsum("tjd,td->tj", y, dout)


def silu_grad(z):
    """d/dz of z sigmoid(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + np.asarray(z, np.float64) * (1.0 - s))


def gelu_tanh_grad(z):
    """d/dz of 0.5 z (1 + tanh(c (z + a z^3))), by the product and chain rules."""
    z = np.asarray(z, dtype=np.float64)
    th = np.tanh(SQRT_2_OVER_PI * (z + GELU_CUBIC * z ** 3))
    return 0.5 * (1.0 + th) + 0.5 * z * (1.0 - th * th) * SQRT_2_OVER_PI * (
        1.0 + 3.0 * GELU_CUBIC * z * z)


def activation_grad(kind: int, z):
    if kind == ACT_SILU:
        return silu_grad(z)
    if kind == ACT_GELU_TANH:
        return gelu_tanh_grad(z)
    raise ValueError(f"unknown activation {kind}")


def glu(gate_up, kind: int):
    """h = act(g) * u for rows gate_up = g | u."""
    gu = np.asarray(gate_up, np.float64)
    I = gu.shape[1] // 2
    return activation(kind, gu[:, :I]) * gu[:, I:]


def glu_backward(gate_up, dh, kind: int):
    """dg = dh u act'(g), du = dh act(g), returned in the gate_up layout."""
    gu = np.asarray(gate_up, np.float64)
    dh = np.asarray(dh, np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    return np.concatenate([dh * u * activation_grad(kind, g), dh * activation(kind, g)], axis=1)


# ---------------------------------------------------------------- permutation
def permutation(ids, E: int):
    """Stable grouping of the flat routes r = t*k + j by expert.

    cnt[e]  = number of routes that chose e
    off     = exclusive prefix sum of cnt (length E+1)
    pos(r)  = off[e_r] + #{r' < r : e_r' = e_r}
    perm[pos(r)] = r, and the inverse pos_of_route[r] = pos(r)
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    R = flat.shape[0]
    cnt = np.zeros(E, dtype=np.int64)
    for r in range(R):
        cnt[flat[r]] += 1
    off = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        off[e + 1] = off[e] + cnt[e]
    seen = np.zeros(E, dtype=np.int64)
    perm = np.zeros(R, dtype=np.int64)
    pos_of_route = np.zeros(R, dtype=np.int64)
    for r in range(R):
        e = flat[r]
        p = off[e] + seen[e]
        seen[e] += 1
        perm[p] = r
        pos_of_route[r] = p
    return cnt, off, perm, pos_of_route


# ------------------------------------------------------------------ experts
def expert_ffn(xt, Wg, Wu, Wd, act: int) -> np.ndarray:
    """One gated expert on one token: Wd (act(Wg x) * (Wu x)), float64."""
    g = Wg @ xt
    u = Wu @ xt
    return Wd @ (activation(act, g) * u)


class WeightSource:
    """Decodes one expert's [out, in] matrices to float64 on demand.

    ``inputs`` is a moe_synth.MoeInputs with numpy arrays (or objects whose
    ``[e]`` indexing yields numpy arrays in storage format).
    """

    def __init__(self, inputs, cache: bool = True):
        from moe_synth.configs import WF_BF16, WF_U4, DT_BF16
        self.inp = inputs
        self.cfg = inputs.cfg
        self.wbf16 = self.cfg.weight_format == WF_BF16
        self.u4 = self.cfg.weight_format == WF_U4
        self.rbf16 = self.cfg.router_dtype == DT_BF16
        self.xbf16 = self.cfg.act_dtype == DT_BF16
        self._cache = {} if cache else None

    def _mat(self, which, e):
        key = (which, e)
        if self._cache is not None and key in self._cache:
            return self._cache[key]
        w = getattr(self.inp, which)
        if self.u4:
            m = u4_dequant(np.asarray(w.codes[e]), np.asarray(w.scales[e]),
                           np.asarray(w.mins[e]), w.K, w.group)
        else:
            m = decode_matrix(np.asarray(w[e]), self.wbf16)
        if self._cache is not None:
            self._cache[key] = m
        return m

    def expert(self, e):
        return self._mat("gate", e), self._mat("up", e), self._mat("down", e)

    def x_row(self, t):
        return decode_matrix(np.asarray(self.inp.x[t]), self.xbf16)

    def router(self):
        return decode_matrix(np.asarray(self.inp.router[:]), self.rbf16)

    def router_bias(self):
        b = self.inp.router_bias
        return None if b is None else np.asarray(b[:], dtype=np.float32).astype(np.float64)

    def shared(self):
        key = ("shared", 0)
        if self._cache is not None and key in self._cache:
            return self._cache[key]
        i = self.inp
        v = (decode_matrix(np.asarray(i.shared_gate_inp[:]), self.rbf16),
             decode_matrix(np.asarray(i.shared_gate[:]), self.wbf16),
             decode_matrix(np.asarray(i.shared_up[:]), self.wbf16),
             decode_matrix(np.asarray(i.shared_down[:]), self.wbf16))
        if self._cache is not None:
            self._cache[key] = v
        return v


def shared_expert(xt, w_sg, Wsg, Wsu, Wsd):
    """sigmoid(x . w_sg) * Wsd (silu(Wsg x) * (Wsu x))  (hf2q op order 3-9)."""
    s = sigmoid(float(xt @ w_sg))
    return s * (Wsd @ (silu(Wsg @ xt) * (Wsu @ xt))), s


def moe_ffn(inputs, tokens=None, normalize: bool = True, src: WeightSource = None,
            gating: int = GATING_SOFTMAX, scale: float = 1.0, pre_norm=None, residual=None,
            expert_scale=None):
    """The whole layer for the given token ids (all tokens by default).

    Returns dict with out [n, H] float64, ids [n, k], w [n, k] float64,
    logits [n, E] float64 and (when present) shared gate values [n].
    ``pre_norm`` = (norm_weight [H], eps) runs the layer on the RMSNorm of
    x, stored in the activation type; ``residual`` [T, H] is added to out
    (hf2q's residual folded into the final reduce); ``expert_scale`` [E] is
    the per-expert routing scale of ``route``.
    """
    cfg = inputs.cfg
    src = src or WeightSource(inputs)
    toks = list(range(cfg.T)) if tokens is None else list(tokens)
    X = np.stack([src.x_row(t) for t in toks]) if toks else np.zeros((0, cfg.H))
    if pre_norm is not None and toks:
        nw, eps = pre_norm
        X = round_to_act(rms_norm(X, nw, eps), cfg.act_dtype == 1)
    logits = router_logits(X, src.router(), src.router_bias())
    ids, w = route(logits, cfg.k, normalize, gating, scale, expert_scale)
    out = np.zeros((len(toks), cfg.H), dtype=np.float64)
    sgate = np.zeros(len(toks), dtype=np.float64)
    for n in range(len(toks)):
        for j in range(cfg.k):
            Wg, Wu, Wd = src.expert(int(ids[n, j]))
            out[n] += w[n, j] * expert_ffn(X[n], Wg, Wu, Wd, cfg.act)
        if cfg.shared:
            w_sg, Wsg, Wsu, Wsd = src.shared()
            ys, s = shared_expert(X[n], w_sg, Wsg, Wsu, Wsd)
            out[n] += ys
            sgate[n] = s
        if residual is not None:
            out[n] += np.asarray(residual[toks[n]], dtype=np.float64)
    return {"out": out, "ids": ids, "w": w, "logits": logits, "shared_gate": sgate,
            "tokens": toks}
