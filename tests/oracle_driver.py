"""Test-side drivers of the CPU oracle for large workloads (test
infrastructure only).

``layer_by_expert`` is oracle.moe_ffn for a sample of tokens with each
expert's matrices decoded once for every sampled token that chose it
(moe_ffn decodes them per token, which is too slow at the largest shapes).
It calls the oracle's own steps (router_logits, route, expert_ffn,
shared_expert) with the same arguments and sums in the same order (slots
in order, then the shared expert, then the residual), so its result is
bit-identical to moe_ffn's; a CPU test checks that.

``tile_covering_tokens`` picks the tokens whose outputs a full-size parity
test compares: tokens from route tiles spread over the whole tile list of
the prefill grouped GEMMs (so every XCD's share of tiles is sampled), from
the last, ragged tile of the most loaded expert, and from the shared
expert's last tile.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O


def layer_by_expert(inp, tokens, normalize=True, gating=0, scale=1.0, pre_norm=None,
                    residual=None, expert_scale=None, src=None):
    cfg = inp.cfg
    src = src or O.WeightSource(inp, cache=False)
    toks = list(tokens)
    X = np.stack([src.x_row(t) for t in toks]) if toks else np.zeros((0, cfg.H))
    if pre_norm is not None and toks:
        nw, eps = pre_norm
        X = O.round_to_act(O.rms_norm(X, nw, eps), cfg.act_dtype == 1)
    logits = O.router_logits(X, src.router(), src.router_bias())
    ids, w = O.route(logits, cfg.k, normalize, gating, scale, expert_scale)
    Y = np.zeros((len(toks), cfg.k, cfg.H), dtype=np.float64)
    for e in np.unique(ids):
        Wg, Wu, Wd = src.expert(int(e))
        for n, j in zip(*np.nonzero(ids == e)):
            Y[n, j] = O.expert_ffn(X[n], Wg, Wu, Wd, cfg.act)
    shared = src.shared() if cfg.shared else None
    out = np.zeros((len(toks), cfg.H), dtype=np.float64)
    for n in range(len(toks)):
        for j in range(cfg.k):
            out[n] += w[n, j] * Y[n, j]
        if shared is not None:
            ys, _ = O.shared_expert(X[n], *shared)
            out[n] += ys
        if residual is not None:
            out[n] += np.asarray(residual[toks[n]], dtype=np.float64)
    return out


def tile_covering_tokens(ids, E, k, T, shared, tile=256, spread=24):
    """Tokens covering the grouped GEMMs' route tiles.

    The tile list holds, expert by expert, ceil(count / tile) tiles of
    consecutive grouped routes, then (with a shared expert) ceil(T / tile)
    tiles of all tokens in order; the GEMMs deal it to the XCDs in equal
    consecutive ranges.  Picked: the last route of tiles evenly spaced over
    the list (first and last included) until `spread` distinct tokens are
    in (or every tile is), the first and last route of the most loaded
    expert's last tile, and the last token of the shared expert's first and
    last tiles."""
    cnt, off, perm, _ = O.permutation(ids, E)
    tiles = []   # (start position, length) in the grouped route order; shared: token ranges
    for e in range(E):
        for i in range((int(cnt[e]) + tile - 1) // tile):
            s = int(off[e]) + i * tile
            tiles.append(("r", s, min(tile, int(cnt[e]) - i * tile)))
    if shared:
        for i in range((T + tile - 1) // tile):
            tiles.append(("s", i * tile, min(tile, T - i * tile)))
    toks = set()
    # tiles of one token can coincide: widen the spread until `spread`
    # distinct tokens are in (or every tile is)
    m = min(spread, len(tiles))
    while True:
        for q in np.linspace(0, len(tiles) - 1, m).round().astype(int):
            kind, s, n = tiles[q]
            toks.add(int(perm[s + n - 1]) // k if kind == "r" else s + n - 1)
        if len(toks) >= spread or m >= len(tiles):
            break
        m = min(len(tiles), m + (spread - len(toks)) + 1)
    hot = int(np.argmax(cnt))
    last = (int(cnt[hot]) - 1) // tile
    s = int(off[hot]) + last * tile
    toks.add(int(perm[s]) // k)
    toks.add(int(perm[int(off[hot]) + int(cnt[hot]) - 1]) // k)
    if shared:
        toks.add(min(tile, T) - 1)
        toks.add(T - 1)
    return sorted(toks)
