"""Pins for the CPU oracle: values the pages print, closed forms, brute force
on tiny inputs, and special cases that reduce to a dense FFN.  None of these
re-types the oracle's own formulas; each would fail on a plausible mistake
(dropped term, wrong sign, transposed operand, wrong tie rule)."""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from conftest import read_golden_rows
from oracle import moe_oracle as O
from oracle.cases import make_inputs, margin_violations, MARGIN
from moe_synth import (CONFIGS, MoeConfig, MoeInputs, U4Weights, generate,
                       f32_to_bf16_bits, WF_F32, WF_BF16, WF_U4, ACT_SILU,
                       ACT_GELU_TANH, DT_F32, DT_BF16)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------- activations
def test_silu_known_values_from_page():
    for g, u, exp in read_golden_rows("silu_known_values.txt"):
        got = O.silu(float(g)) * float(u)
        assert abs(got - float(exp)) < 1e-5


def test_gelu_tanh_points_from_page():
    for z, exp, tol in read_golden_rows("gelu_tanh_points.txt"):
        assert abs(float(O.gelu_tanh(float(z))) - float(exp)) <= float(tol)


def test_activations_match_torch_library():
    z = np.linspace(-12, 12, 2001)
    tz = torch.from_numpy(z)
    np.testing.assert_allclose(O.silu(z), F.silu(tz).numpy(), rtol=1e-14, atol=1e-300)
    # torch's tanh GELU uses sqrt(2/pi) to full precision; the page prints
    # 0.7978845608, so the two differ by < 3e-11 relative in the constant.
    np.testing.assert_allclose(O.gelu_tanh(z), F.gelu(tz, approximate="tanh").numpy(),
                               rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(O.sigmoid(z), torch.sigmoid(tz).numpy(), rtol=1e-14)


# ------------------------------------------------------------------ routing
def test_softmax_topk_basic_from_page():
    rows = {r[0]: r[1:] for r in read_golden_rows("softmax_topk_basic.txt")}
    logits = np.array([float(v) for v in rows["logits"]])
    k = int(rows["k"][0])
    ids, w = O.route(logits[None, :], k)
    assert ids[0].tolist() == [int(v) for v in rows["ids"]]
    assert abs(w.sum() - 1.0) < float(rows["sum_tol"][0])


def test_zero_logits_take_lowest_indices():
    for E, k in [(8, 2), (128, 8), (256, 8), (5, 5)]:
        ids, w = O.route(np.zeros((1, E)), k)
        assert ids[0].tolist() == list(range(k))
        np.testing.assert_allclose(w[0], np.full(k, 1.0 / k), rtol=0, atol=1e-15)


def _brute_best_set(logits, k):
    """Max-sum k-subset; among equal sums the lexicographically lowest."""
    best, best_sum = None, -math.inf
    for comb in itertools.combinations(range(len(logits)), k):
        s = sum(logits[i] for i in comb)
        if s > best_sum:
            best, best_sum = comb, s
    return best


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 2), (8, 4), (7, 7)])
def test_route_brute_force_random(E, k):
    rng = np.random.default_rng(1000 + 10 * E + k)
    for _ in range(50):
        l = rng.normal(size=E)
        ids, w = O.route(l[None, :], k)
        assert sorted(ids[0].tolist()) == list(_brute_best_set(l, k))
        # slots are in descending probability
        assert all(l[ids[0][j]] > l[ids[0][j + 1]] for j in range(k - 1))


def test_route_brute_force_integer_ties():
    # small integer logits produce many exact ties: the set must be the
    # lexicographically lowest max-sum set, and equal values appear in
    # ascending index order within the slots
    rng = np.random.default_rng(7)
    for _ in range(300):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-2, 3, size=E).astype(np.float64)
        ids, w = O.route(l[None, :], k)
        got = ids[0].tolist()
        assert sorted(got) == list(_brute_best_set(l.tolist(), k))
        for j in range(k - 1):
            a, b = got[j], got[j + 1]
            assert l[a] > l[b] or (l[a] == l[b] and a < b)


def test_route_weights_sum_to_one_and_match_winner_softmax():
    rng = np.random.default_rng(3)
    L = rng.normal(size=(64, 128)) * 3
    ids, w = O.route(L, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # renormalised top-k == softmax taken over the k winners only
    for t in range(L.shape[0]):
        ref = scipy.special.softmax(L[t, ids[t]])
        np.testing.assert_allclose(w[t], ref, rtol=1e-14, atol=0)


def test_route_unnormalised_is_softmax_of_all():
    rng = np.random.default_rng(4)
    L = rng.normal(size=(16, 32))
    ids, w = O.route(L, 4, normalize=False)
    P = scipy.special.softmax(L, axis=1)
    for t in range(16):
        np.testing.assert_allclose(w[t], P[t, ids[t]], rtol=1e-14)


def test_route_shift_invariance():
    rng = np.random.default_rng(5)
    L = rng.normal(size=(32, 64))
    ids0, w0 = O.route(L, 8)
    ids1, w1 = O.route(L + 17.25, 8)   # exact shift in fp64 for these values
    assert (ids0 == ids1).all()
    np.testing.assert_allclose(w0, w1, rtol=1e-13)


# ----------------------------------------------- sigmoid gating, weight scale
def test_sigmoid_gating_selects_like_softmax():
    # both scores increase with the logit: same experts, same slot order,
    # ties (equal logits) still to the lower index
    rng = np.random.default_rng(41)
    for _ in range(200):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, size=E).astype(np.float64) * 0.5
        a, _ = O.route(l[None, :], k)
        b, _ = O.route(l[None, :], k, gating=O.GATING_SIGMOID)
        assert (a == b).all()


def test_one_expert_weight_is_one_under_either_gating():
    # the dense-layer note: softmax of one logit is 1, and sigmoid followed
    # by renormalisation divides the selected score by itself
    for g in (O.GATING_SOFTMAX, O.GATING_SIGMOID):
        for l in (-40.0, -1.5, 0.0, 2.25, 30.0):
            ids, w = O.route(np.array([[l]]), 1, gating=g)
            assert ids[0, 0] == 0 and w[0, 0] == 1.0


def test_sigmoid_gating_worked_values():
    # logits (ln 3, 0, -ln 3): sigmoid scores 3/4, 1/2, 1/4
    l = np.array([[math.log(3.0), 0.0, -math.log(3.0)]])
    ids, w = O.route(l, 2, gating=O.GATING_SIGMOID)
    assert ids[0].tolist() == [0, 1]
    np.testing.assert_allclose(w[0], [0.6, 0.4], rtol=1e-15)          # 0.75/1.25, 0.5/1.25
    ids, w = O.route(l, 2, normalize=False, gating=O.GATING_SIGMOID)
    np.testing.assert_allclose(w[0], [0.75, 0.5], rtol=1e-15)
    ids, w = O.route(l, 2)                                             # softmax: 3:1 of e^l
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-15)


def test_sigmoid_unnormalised_is_library_expit():
    rng = np.random.default_rng(42)
    L = rng.normal(size=(16, 40)) * 2
    ids, w = O.route(L, 6, normalize=False, gating=O.GATING_SIGMOID)
    for t in range(16):
        np.testing.assert_allclose(w[t], scipy.special.expit(L[t, ids[t]]), rtol=1e-14)
    ids, w = O.route(L, 6, gating=O.GATING_SIGMOID)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # unlike softmax, sigmoid weights move when every logit shifts by a constant
    _, w2 = O.route(L + 1.0, 6, gating=O.GATING_SIGMOID)
    assert np.abs(w2 - w).max() > 1e-3


def test_weight_scale_worked_values_and_routed_sum_only():
    # logits (ln 3, 0): softmax 3/4, 1/4; a scale of 2.5 gives 1.875, 0.625
    l = np.array([[math.log(3.0), 0.0]])
    _, w = O.route(l, 2, scale=2.5)
    np.testing.assert_allclose(w[0], [1.875, 0.625], rtol=1e-15)
    # sigmoid scores 3/4, 1/2, raw, times 2.5
    _, w = O.route(l, 2, normalize=False, gating=O.GATING_SIGMOID, scale=2.5)
    np.testing.assert_allclose(w[0], [1.875, 1.25], rtol=1e-15)
    # renormalised weights then sum to the scale, whatever the logits
    rng = np.random.default_rng(44)
    _, w = O.route(rng.normal(size=(32, 16)) * 3, 4, scale=2.5)
    np.testing.assert_allclose(w.sum(axis=1), 2.5, rtol=0, atol=1e-13)
    for g in (O.GATING_SOFTMAX, O.GATING_SIGMOID):
        base = O.moe_ffn(_tiny_inputs(seed=43, shared=True, T=4), gating=g)
        sc = O.moe_ffn(_tiny_inputs(seed=43, shared=True, T=4), gating=g, scale=2.5)
        routed = O.moe_ffn(_tiny_inputs(seed=43, shared=False, T=4), gating=g)["out"]
        # the shared expert's contribution is untouched by the scale
        np.testing.assert_allclose(sc["out"] - base["out"], 1.5 * routed, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("act", [ACT_SILU, ACT_GELU_TANH])
def test_weight_scale_single_expert_is_scaled_dense_ffn(act):
    # one expert, top-1: the routed part is the dense gated FFN, computed
    # here with torch's linear layers, times the scale
    inp = _tiny_inputs(E=1, k=1, act=act, seed=45)
    r = O.moe_ffn(inp, scale=-0.75)
    x = torch.from_numpy(inp.x).double()
    g = F.linear(x, torch.from_numpy(inp.gate[0]).double())
    u = F.linear(x, torch.from_numpy(inp.up[0]).double())
    a = F.silu(g) if act == ACT_SILU else F.gelu(g, approximate="tanh")
    ref = -0.75 * F.linear(a * u, torch.from_numpy(inp.down[0]).double()).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------ per-expert scale
def test_expert_scale_worked_values():
    # logits (ln 3, 0): softmax 3/4, 1/4.  Scales (2, 1): scaled scores
    # 3/2, 1/4, renormalised 6/7, 1/7; raw 3/2, 1/4; times a weight scale of
    # 2: 12/7, 2/7
    l = np.array([[math.log(3.0), 0.0]])
    es = np.array([2.0, 1.0])
    ids, w = O.route(l, 2, expert_scale=es)
    assert ids[0].tolist() == [0, 1]
    np.testing.assert_allclose(w[0], [6 / 7, 1 / 7], rtol=1e-15)
    _, w = O.route(l, 2, normalize=False, expert_scale=es)
    np.testing.assert_allclose(w[0], [1.5, 0.25], rtol=1e-15)
    _, w = O.route(l, 2, expert_scale=es, scale=2.0)
    np.testing.assert_allclose(w[0], [12 / 7, 2 / 7], rtol=1e-15)
    # sigmoid scores 3/4, 1/2 with scales (1, 3): 3/4, 3/2 -> 1/3, 2/3
    _, w = O.route(l, 2, gating=O.GATING_SIGMOID, expert_scale=np.array([1.0, 3.0]))
    np.testing.assert_allclose(w[0], [1 / 3, 2 / 3], rtol=1e-15)


def test_expert_scale_ones_is_plain_routing_and_k1_weight_is_one():
    rng = np.random.default_rng(46)
    L = rng.normal(size=(24, 32)) * 2
    for g in (O.GATING_SOFTMAX, O.GATING_SIGMOID):
        for nrm in (True, False):
            a = O.route(L, 5, nrm, g)
            b = O.route(L, 5, nrm, g, expert_scale=np.ones(32))
            assert (a[0] == b[0]).all()
            np.testing.assert_array_equal(a[1], b[1])
    # renormalising one selected expert's scaled score gives exactly 1
    es = rng.uniform(0.5, 1.5, size=32)
    for g in (O.GATING_SOFTMAX, O.GATING_SIGMOID):
        _, w = O.route(L, 1, gating=g, expert_scale=es)
        assert (w == 1.0).all()


def test_expert_scale_does_not_change_selection():
    # the scale applies to the gathered winners: a large scale on an
    # expert with a small logit does not select it
    rng = np.random.default_rng(47)
    L = rng.normal(size=(40, 16))
    es = np.ones(16)
    es[int(np.argmin(L[0]))] = 1e6
    a, _ = O.route(L, 4)
    b, wb = O.route(L, 4, expert_scale=es)
    assert (a == b).all()
    # renormalised weights are proportional to p_e * s_e over the winners
    P = scipy.special.softmax(L, axis=1)
    for t in range(40):
        ref = P[t, b[t]] * es[b[t]]
        np.testing.assert_allclose(wb[t], ref / ref.sum(), rtol=1e-13)


def test_expert_scale_equals_scaled_down_weights_without_renormalisation():
    # unnormalised weights enter the output linearly: scaling expert e's
    # weight by 2^m equals scaling its down matrix by 2^m (exact in f32)
    es = np.array([2.0, 0.5, 4.0, 0.25], dtype=np.float32)
    a = O.moe_ffn(_tiny_inputs(seed=48, T=6), normalize=False, expert_scale=es)
    inp = _tiny_inputs(seed=48, T=6)
    inp.down = inp.down * es[:, None, None]
    b = O.moe_ffn(inp, normalize=False)
    assert (a["ids"] == b["ids"]).all()
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-15)


# ------------------------------------------------- pre-FFN RMSNorm, residual
def test_rms_norm_worked_value_and_library():
    # [3, 4]: mean square 12.5, so x / sqrt(12.5) = x * sqrt(2) / 5
    np.testing.assert_allclose(O.rms_norm([[3.0, 4.0]], [1.0, 1.0], 0.0),
                               [[3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5]], rtol=1e-15)
    rng = np.random.default_rng(51)
    X = rng.normal(size=(7, 96)) * 3
    w = rng.uniform(0.5, 1.5, size=96)
    ref = F.rms_norm(torch.from_numpy(X), (96,), torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rms_norm(X, w, 1e-5), ref, rtol=1e-13, atol=1e-15)
    # invariant under a positive scale of the row when eps is 0
    np.testing.assert_allclose(O.rms_norm(X * 7.5, w, 0.0), O.rms_norm(X, w, 0.0), rtol=1e-13)


def test_round_to_act_matches_library_casts():
    rng = np.random.default_rng(52)
    X = rng.normal(size=(5, 64)) * 10
    t = torch.from_numpy(X)
    np.testing.assert_array_equal(O.round_to_act(X, False), t.float().double().numpy())
    np.testing.assert_array_equal(O.round_to_act(X, True),
                                  t.float().bfloat16().double().numpy())


def test_pre_norm_layer_runs_on_normalised_rows():
    inp = _tiny_inputs(seed=53, T=4, H=32)
    nw = np.linspace(0.6, 1.4, 32)
    normed = O.round_to_act(O.rms_norm(inp.x, nw, 1e-6), False)
    direct = _tiny_inputs(seed=53, T=4, H=32)
    direct.x = normed.astype(np.float32)      # exact: normed already holds float32 values
    np.testing.assert_allclose(O.moe_ffn(inp, pre_norm=(nw, 1e-6))["out"],
                               O.moe_ffn(direct)["out"], rtol=1e-13, atol=1e-15)
    # a positive rescale of x leaves the normalised layer unchanged (up to f32 rounding)
    big = _tiny_inputs(seed=53, T=4, H=32)
    big.x = big.x * np.float32(16.0)          # exact power of two
    np.testing.assert_allclose(O.moe_ffn(big, pre_norm=(nw, 0.0))["out"],
                               O.moe_ffn(inp, pre_norm=(nw, 0.0))["out"], rtol=1e-12, atol=1e-14)


def test_residual_is_added_to_out():
    inp = _tiny_inputs(seed=54, T=3, shared=True)
    r = np.random.default_rng(55).normal(size=(3, 16))
    a = O.moe_ffn(inp)["out"]
    b = O.moe_ffn(inp, residual=r)["out"]
    np.testing.assert_allclose(b - a, r, rtol=0, atol=1e-14)
    c = O.moe_ffn(inp, residual=-a)["out"]    # the residual cancels the layer
    np.testing.assert_allclose(c, 0.0, atol=1e-14)


# ----------------------------------------------------------------- backward
def _fd(f, x, eps=1e-6):
    """Central differences of the scalar f at x, every element."""
    x = np.array(x, dtype=np.float64)
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        g[i] = (f(xp) - f(xm)) / (2 * eps)
    return g


def test_weighted_sum_backward_finite_differences():
    # the page's falsifier: L = sum(out * seed); dL/dy and dL/dw by differences
    rng = np.random.default_rng(61)
    T, k, H = 3, 4, 7
    y = rng.normal(size=(T, k, H))
    w = rng.uniform(0.2, 1.0, size=(T, k))
    seed = rng.normal(size=(T, H))
    dy, dw = O.weighted_sum_backward(w, y, seed)
    np.testing.assert_allclose(dy, _fd(lambda v: (O.weighted_sum(w, v) * seed).sum(), y),
                               rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(dw, _fd(lambda v: (O.weighted_sum(v, y) * seed).sum(), w),
                               rtol=1e-7, atol=1e-8)


@pytest.mark.parametrize("act", [ACT_SILU, ACT_GELU_TANH])
def test_glu_backward_finite_differences_and_autograd(act):
    rng = np.random.default_rng(62 + act)
    R, I = 4, 5
    gu = rng.normal(size=(R, 2 * I)) * 3
    seed = rng.normal(size=(R, I))
    got = O.glu_backward(gu, seed, act)
    np.testing.assert_allclose(got, _fd(lambda v: (O.glu(v, act) * seed).sum(), gu),
                               rtol=1e-6, atol=1e-8)
    t = torch.from_numpy(gu).requires_grad_(True)
    g, u = t[:, :I], t[:, I:]
    a = F.silu(g) if act == ACT_SILU else F.gelu(g, approximate="tanh")
    (a * u * torch.from_numpy(seed)).sum().backward()
    np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-8, atol=1e-12)


def test_glu_backward_asymptotics_from_page():
    rows = {r[0]: [float(v) for v in r[1:]] for r in read_golden_rows("glu_backward_asymptotics.txt")}
    gu = np.array([rows["g"] + rows["u"]])
    d = np.array([rows["d"]])
    out = O.glu_backward(gu, d, ACT_GELU_TANH)[0]
    tol = np.array(rows["tol"])
    assert (np.abs(out[:3] - rows["dg"]) <= tol).all()
    assert (np.abs(out[3:] - rows["du"]) <= tol).all()


def test_router_logits_transpose_and_bias():
    # l[t, e] = x_t . Wr[e]: a rectangular check that catches a transposed Wr
    x = np.array([[1.0, 2.0, 3.0]])
    Wr = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    np.testing.assert_array_equal(O.router_logits(x, Wr), [[1.0, 3.0]])
    np.testing.assert_array_equal(O.router_logits(x, Wr, np.array([0.5, -4.0])), [[1.5, -1.0]])


# -------------------------------------------------------------- permutation
def test_permutation_hand_example():
    ids = np.array([[2, 0], [0, 1], [2, 1]])      # routes 0..5 -> experts 2,0,0,1,2,1
    cnt, off, perm, pos = O.permutation(ids, 4)
    assert cnt.tolist() == [2, 2, 2, 0]
    assert off.tolist() == [0, 2, 4, 6, 6]
    assert perm.tolist() == [1, 2, 3, 5, 0, 4]
    assert pos.tolist() == [4, 0, 1, 2, 5, 3]


@pytest.mark.parametrize("T,k,E,skew", [(1, 8, 128, False), (37, 8, 256, True),
                                         (300, 2, 8, False), (64, 8, 256, False)])
def test_permutation_properties(T, k, E, skew):
    rng = np.random.default_rng(T * 31 + E)
    if skew:
        p = 1.0 / np.arange(1, E + 1)
        p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p if skew else None)
                    for _ in range(T)])
    cnt, off, perm, pos = O.permutation(ids, E)
    flat = ids.reshape(-1)
    R = flat.size
    assert sorted(perm.tolist()) == list(range(R))                  # bijection
    assert (perm[pos] == np.arange(R)).all()                        # inverse
    assert (np.bincount(flat, minlength=E) == cnt).all()
    assert (perm == np.argsort(flat, kind="stable")).all()          # stable grouping
    for e in range(E):                                              # contiguous blocks
        assert (flat[perm[off[e]:off[e + 1]]] == e).all()


# ----------------------------------------------------------- storage decode
def test_bf16_and_f16_decode_known_patterns():
    b = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x3E20], dtype=np.uint16)
    exp = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.15625]
    np.testing.assert_array_equal(O.bf16_to_f64(b), exp)
    h = np.array([0x3C00, 0x0001, 0x7BFF, 0xC100, 0x2E66], dtype=np.uint16)
    exp = [1.0, 2.0 ** -24, 65504.0, -2.5, 0.0999755859375]
    np.testing.assert_array_equal(O.f16_to_f64(h), exp)


def test_bf16_generator_rounding_matches_torch():
    rng = np.random.default_rng(11)
    v = (rng.normal(size=100000) * rng.choice([1e-3, 1, 1e3], size=100000)).astype(np.float32)
    mine = f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (mine == ref).all()


def test_u4_nibble_order_and_affine_form():
    # byte 0x21 holds element 0 = 1 (low nibble), element 1 = 2 (high nibble)
    codes = np.array([[0x21] + [0xF0] * 15], dtype=np.uint8)        # K = 32
    sc = np.array([[0x3C00]], dtype=np.uint16)                       # 1.0
    mn = np.array([[0xC800]], dtype=np.uint16)                       # -8.0
    w = O.u4_dequant(codes, sc, mn, 32, 32)
    assert w[0, 0] == 1 - 8 and w[0, 1] == 2 - 8
    assert w[0, 2] == 0 - 8 and w[0, 3] == 15 - 8                   # code 0 -> min, 15 -> 15s+min


def test_u4_generated_min_is_minus_eight_scale():
    cfg = MoeConfig(name="u4pin", T=3, H=64, I=64, E=4, k=2, weight_format=WF_U4)
    inp = generate(cfg)
    for wt in (inp.gate, inp.up, inp.down):
        s = O.f16_to_f64(wt.scales)
        m = O.f16_to_f64(wt.mins)
        np.testing.assert_array_equal(m, -8.0 * s)
        assert s.min() >= 0.005 - 1e-5 and s.max() <= 0.02 + 1e-5
        full = O.u4_dequant(wt.codes[1], wt.scales[1], wt.mins[1], wt.K, wt.group)
        q = np.empty((wt.codes.shape[1], wt.K))
        q[:, 0::2] = wt.codes[1] & 15
        q[:, 1::2] = wt.codes[1] >> 4
        np.testing.assert_array_equal(full, (q - 8) * np.repeat(s[1], 32, axis=1))


# ------------------------------------------------------------ whole layer
def _tiny_inputs(E=4, k=2, H=16, I=8, T=5, act=ACT_SILU, seed=0, shared=False, Is=8):
    rng = np.random.default_rng(seed)
    cfg = MoeConfig(name="pin", T=T, H=H, I=I, E=E, k=k, act=act, shared=shared, Is=Is)
    f = lambda *s: rng.normal(size=s).astype(np.float32)
    inp = MoeInputs(cfg, f(T, H), f(E, H), None, f(E, I, H) / 4, f(E, I, H) / 4,
                    f(E, H, I) / 3)
    if shared:
        inp.shared_gate_inp = f(H)
        inp.shared_gate, inp.shared_up, inp.shared_down = f(Is, H) / 4, f(Is, H) / 4, f(H, Is) / 3
    return inp


@pytest.mark.parametrize("act", [ACT_SILU, ACT_GELU_TANH])
def test_single_expert_top1_is_dense_ffn(act):
    inp = _tiny_inputs(E=1, k=1, act=act, seed=21)
    r = O.moe_ffn(inp)
    assert (r["w"] == 1.0).all() and (r["ids"] == 0).all()
    x = torch.from_numpy(inp.x).double()
    g = F.linear(x, torch.from_numpy(inp.gate[0]).double())
    u = F.linear(x, torch.from_numpy(inp.up[0]).double())
    a = F.silu(g) if act == ACT_SILU else F.gelu(g, approximate="tanh")
    ref = F.linear(a * u, torch.from_numpy(inp.down[0]).double()).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-9, atol=1e-12)


def test_zero_expert_weights_give_zero():
    inp = _tiny_inputs(seed=22)
    inp.gate[:] = 0
    inp.up[:] = 0
    inp.down[:] = 0
    assert (O.moe_ffn(inp)["out"] == 0).all()


@pytest.mark.parametrize("act", [ACT_SILU, ACT_GELU_TANH])
def test_identity_experts_give_act_x_times_x(act):
    H = 16
    inp = _tiny_inputs(E=6, k=3, H=H, I=H, act=act, seed=23)
    eye = np.eye(H, dtype=np.float32)
    inp.gate[:] = eye
    inp.up[:] = eye
    inp.down[:] = eye
    x = inp.x.astype(np.float64)
    ref = (F.silu if act == ACT_SILU else (lambda t: F.gelu(t, approximate="tanh")))(
        torch.from_numpy(x)).numpy() * x
    # torch's GELU uses the full sqrt(2/pi); the page prints it to 10 digits
    rtol = 1e-12 if act == ACT_SILU else 1e-9
    np.testing.assert_allclose(O.moe_ffn(inp)["out"], ref, rtol=rtol, atol=1e-14)


def test_basis_vector_input_selects_columns():
    inp = _tiny_inputs(E=5, k=2, seed=24)
    i = 3
    inp.x[:] = 0
    inp.x[:, i] = 1.0
    # router depends on column i only; make it unambiguous
    inp.router[:, i] = np.array([0.3, 2.0, -1.0, 1.1, 0.2], dtype=np.float32)
    r = O.moe_ffn(inp)
    assert r["ids"][0].tolist() == [1, 3]
    ref = np.zeros(inp.cfg.H)
    for j, e in enumerate(r["ids"][0]):
        g = inp.gate[e][:, i].astype(np.float64)
        u = inp.up[e][:, i].astype(np.float64)
        ref += r["w"][0, j] * (inp.down[e].astype(np.float64) @ (O.silu(g) * u))
    np.testing.assert_allclose(r["out"][0], ref, rtol=1e-12)


def test_identical_experts_make_routing_irrelevant():
    inp = _tiny_inputs(E=6, k=3, seed=25)
    for e in range(1, 6):
        inp.gate[e] = inp.gate[0]
        inp.up[e] = inp.up[0]
        inp.down[e] = inp.down[0]
    out = O.moe_ffn(inp)["out"]
    single = _tiny_inputs(E=1, k=1, seed=25)
    single.x, single.gate, single.up, single.down = inp.x, inp.gate[:1], inp.up[:1], inp.down[:1]
    single.router = inp.router[:1]
    np.testing.assert_allclose(out, O.moe_ffn(single)["out"], rtol=1e-12, atol=1e-14)


def test_shared_gate_sigmoid_controls_contribution():
    base = _tiny_inputs(seed=26, shared=True, T=1)
    x = base.x[0].astype(np.float64)
    outs = {}
    for c in (-1000.0, 0.0, 1000.0):
        inp = _tiny_inputs(seed=26, shared=True, T=1)
        inp.shared_gate_inp = (c * x / (x @ x)).astype(np.float64)
        outs[c] = O.moe_ffn(inp)["out"][0]
    routed = _tiny_inputs(seed=26, shared=False, T=1)
    np.testing.assert_allclose(outs[-1000.0], O.moe_ffn(routed)["out"][0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(outs[0.0], 0.5 * (outs[-1000.0] + outs[1000.0]), rtol=1e-12,
                               atol=1e-14)


def _shared_only_inputs(act, seed):
    """Routed experts that contribute nothing (zero down weights), and a
    shared-gate vector whose logit is 1000 for every token (x[:, 0] = 1,
    w_sg = 1000 e_0), so the sigmoid gate is exactly 1 in float64."""
    inp = _tiny_inputs(seed=seed, shared=True, T=3, act=act, Is=12)
    inp.down = np.zeros_like(inp.down)
    inp.x[:, 0] = 1.0
    inp.shared_gate_inp = np.zeros_like(inp.shared_gate_inp)
    inp.shared_gate_inp[0] = 1000.0
    return inp


def _torch_swiglu(inp):
    x = torch.from_numpy(inp.x).double()
    g = F.linear(x, torch.from_numpy(inp.shared_gate).double())
    u = F.linear(x, torch.from_numpy(inp.shared_up).double())
    return F.linear(F.silu(g) * u, torch.from_numpy(inp.shared_down).double()).numpy()


def _shared_pin_holds(act, seed=28):
    inp = _shared_only_inputs(act, seed)
    r = O.moe_ffn(inp)
    if not (r["shared_gate"] == 1.0).all():
        return False
    return np.allclose(r["out"], _torch_swiglu(inp), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("act", [ACT_SILU, ACT_GELU_TANH])
def test_shared_expert_is_a_swiglu_of_its_own_weights(act):
    # the shared expert is SiLU(Wsg x) * (Wsu x) through Wsd, whatever the
    # routed experts' activation (an independent torch computation)
    assert _shared_pin_holds(act)


def test_shared_expert_pin_catches_planted_mistakes(monkeypatch):
    # plant plausible mistakes in the oracle's shared expert: each must make
    # the pin above fail
    def swapped(xt, w_sg, Wsg, Wsu, Wsd):
        s = O.sigmoid(float(xt @ w_sg))
        return s * (Wsd @ (O.silu(Wsu @ xt) * (Wsg @ xt))), s

    def gelu_shared(xt, w_sg, Wsg, Wsu, Wsd):
        s = O.sigmoid(float(xt @ w_sg))
        return s * (Wsd @ (O.gelu_tanh(Wsg @ xt) * (Wsu @ xt))), s

    def transposed_down(xt, w_sg, Wsg, Wsu, Wsd):
        s = O.sigmoid(float(xt @ w_sg))
        h = O.silu(Wsg @ xt) * (Wsu @ xt)
        return s * (Wsd.reshape(Wsd.shape[1], Wsd.shape[0]).T @ h), s

    def ungated(xt, w_sg, Wsg, Wsu, Wsd):
        return 0.5 * (Wsd @ (O.silu(Wsg @ xt) * (Wsu @ xt))), 0.5

    for bad in (swapped, gelu_shared, transposed_down, ungated):
        monkeypatch.setattr(O, "shared_expert", bad)
        assert not _shared_pin_holds(ACT_SILU), bad.__name__
    monkeypatch.undo()
    assert _shared_pin_holds(ACT_SILU)


def test_down_scaling_and_token_permutation():
    inp = _tiny_inputs(seed=27, T=6)
    out = O.moe_ffn(inp)["out"]
    inp2 = _tiny_inputs(seed=27, T=6)
    inp2.down = inp2.down * np.float32(4.0)           # exact power-of-two scaling
    np.testing.assert_allclose(O.moe_ffn(inp2)["out"], 4.0 * out, rtol=1e-15, atol=0)
    inp3 = _tiny_inputs(seed=27, T=6)
    order = np.array([3, 0, 5, 1, 4, 2])
    inp3.x = inp3.x[order]
    np.testing.assert_allclose(O.moe_ffn(inp3)["out"], out[order], rtol=1e-15, atol=0)


def test_u4_layer_equals_f32_layer_on_dequantised_weights():
    cfg = MoeConfig(name="u4eq", T=3, H=64, I=64, E=4, k=2, weight_format=WF_U4)
    inp = generate(cfg)
    r4 = O.moe_ffn(inp)
    cf = MoeConfig(name="f32eq", T=3, H=64, I=64, E=4, k=2, weight_format=WF_F32)
    deq = lambda w: np.stack([O.u4_dequant(w.codes[e], w.scales[e], w.mins[e], w.K, w.group)
                              for e in range(4)]).astype(np.float32)
    inpf = MoeInputs(cf, inp.x, inp.router, None, deq(inp.gate), deq(inp.up), deq(inp.down))
    rf = O.moe_ffn(inpf)
    assert (r4["ids"] == rf["ids"]).all()
    assert (r4["out"] == rf["out"]).all()      # (code-8)*scale is exact in f32


def test_bf16_layer_decodes_storage_exactly():
    cfg = MoeConfig(name="bfeq", T=3, H=32, I=16, E=4, k=2, weight_format=WF_BF16,
                    act_dtype=DT_BF16, router_dtype=DT_BF16)
    inp = generate(cfg)
    rb = O.moe_ffn(inp)
    up = lambda a: (a.astype(np.uint32) << 16).view(np.float32)   # widen bits independently
    cf = MoeConfig(name="f", T=3, H=32, I=16, E=4, k=2)
    inpf = MoeInputs(cf, up(inp.x), up(inp.router), None, up(inp.gate), up(inp.up), up(inp.down))
    assert (O.moe_ffn(inpf)["out"] == rb["out"]).all()


# ------------------------------------------------------- inputs and margins
def test_margin_enforced_on_small_workloads():
    for name in ["tiny_f32"]:
        inp = make_inputs(CONFIGS[name])
        L = O.router_logits(inp.x.astype(np.float64), inp.router.astype(np.float64))
        assert margin_violations(L, inp.cfg.k) == []
    cfg = CONFIGS["prefill_skew_t16384"]
    small = MoeConfig(name="skew_small", T=64, H=64, I=32, E=256, k=8, shared=True, Is=32,
                      weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16,
                      bias=cfg.bias, seed_index=9)
    inp = make_inputs(small)
    L = O.router_logits(O.bf16_to_f64(inp.x), O.bf16_to_f64(inp.router), inp.router_bias)
    assert margin_violations(L, small.k) == []
    # the skew bias makes expert 0 the most loaded
    ids, _ = O.route(L, small.k)
    assert np.bincount(ids.reshape(-1), minlength=256).argmax() == 0


def test_margin_check_detects_close_logits():
    L = np.array([[3.0, 2.0, 2.0 + 0.5 * MARGIN, -1.0], [3.0, 2.0, 1.0, 0.0]])
    assert margin_violations(L, 2) == [0]
    assert margin_violations(L, 1) == []


# ------------------------------------------- the test-side oracle driver
def test_layer_by_expert_is_bit_identical_to_oracle():
    from oracle_driver import layer_by_expert
    from moe_synth import expert_scale_values, residual_values, norm_weight_values
    cfg = MoeConfig(name="drv", T=9, H=64, I=32, E=8, k=3, act=ACT_GELU_TANH,
                    weight_format=WF_BF16, act_dtype=DT_BF16, router_dtype=DT_BF16, shared=True,
                    Is=32, seed_index=90)
    inp = make_inputs(cfg)
    es = expert_scale_values(cfg)
    res = residual_values(cfg)
    pn = (norm_weight_values(cfg), 1e-5)
    toks = [8, 0, 3, 5]
    for kw in (dict(), dict(expert_scale=es, gating=1, scale=2.0), dict(residual=res),
               dict(pre_norm=pn, normalize=False)):
        a = O.moe_ffn(inp, tokens=toks, **kw)["out"]
        b = layer_by_expert(inp, toks, **kw)
        np.testing.assert_array_equal(a, b)


def test_tile_covering_tokens_spread_and_special_tiles():
    from oracle_driver import tile_covering_tokens
    rng = np.random.default_rng(91)
    T, E, k = 3000, 16, 2
    # skewed expert choice: expert 0 far more often, so it has a ragged last tile
    ids = np.stack([rng.choice(E, size=k, replace=False, p=np.r_[0.4, np.full(E - 1, 0.6 / 15)])
                    for _ in range(T)])
    toks = tile_covering_tokens(ids, E, k, T, shared=True, tile=256, spread=12)
    assert len(toks) >= 12 and all(0 <= t < T for t in toks)
    cnt, off, perm, _ = O.permutation(ids, E)
    # the last grouped route of the whole list and the shared expert's last token
    assert int(perm[-1]) // k in toks or T - 1 in toks
    assert T - 1 in toks
    # the hot expert's last route
    assert int(perm[int(off[0]) + int(cnt[0]) - 1]) // k in toks
