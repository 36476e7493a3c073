"""Test cases: seeded inputs with a guaranteed top-k logit margin.

TEST INFRASTRUCTURE ONLY (see moe_oracle.py).

A parity test compares expert ids bit for bit, so no token may have two of
its top k+1 router logits closer than ``MARGIN``: rounding differences
between the float64 oracle and the float32 device logits (about 1e-6 at
these sizes) could otherwise swap two experts.  Tokens that violate the
margin get their x row redrawn from the next generator stream, until all
pass.  The logits used for the check are the oracle's.
"""
from __future__ import annotations

import numpy as np

from moe_synth import generate, x_rows, DT_BF16
from . import moe_oracle as O

MARGIN = 1e-3


def _x_host(inp):
    x = inp.x
    if inp.backend == "numpy":
        return x
    import torch
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def _router_host(inp):
    r = inp.router
    if inp.backend == "numpy":
        return r
    import torch
    if r.dtype == torch.bfloat16:
        return r.view(torch.int16).cpu().numpy().view(np.uint16)
    return r.cpu().numpy()


def margin_violations(logits: np.ndarray, k: int, margin: float = MARGIN):
    """Token ids whose sorted top-(k+1) logits have a gap below ``margin``."""
    bad = []
    E = logits.shape[1]
    m = min(k + 1, E)
    for t in range(logits.shape[0]):
        top = np.sort(logits[t])[::-1][:m]
        if m > 1 and np.min(top[:-1] - top[1:]) < margin:
            bad.append(t)
    return bad


def enforce_margin(inp, margin: float = MARGIN, max_attempts: int = 64, xform=None):
    """Redraw offending x rows in place; returns the number of redraws.

    ``xform`` maps decoded x rows to the router's input when the layer
    transforms x first (the pre-FFN RMSNorm)."""
    xform = xform or (lambda X: X)
    cfg = inp.cfg
    xbf = cfg.act_dtype == DT_BF16
    rbf = cfg.router_dtype == DT_BF16
    Wr = O.decode_matrix(_router_host(inp), rbf)
    b = inp.router_bias
    if b is not None and inp.backend != "numpy":
        b = b.cpu().numpy()
    X = O.decode_matrix(_x_host(inp), xbf)
    bad = margin_violations(O.router_logits(xform(X), Wr, b), cfg.k, margin)
    redraws = 0
    attempt = 1
    while bad:
        if attempt > max_attempts:
            raise RuntimeError(f"could not reach margin for tokens {bad[:8]}")
        rows = x_rows(cfg, bad, attempt, backend=inp.backend,
                      device=None if inp.backend == "numpy" else inp.x.device)
        if inp.backend == "numpy":
            inp.x[bad] = rows
            Xb = O.decode_matrix(rows, xbf)
        else:
            import torch
            idx = torch.tensor(bad, device=inp.x.device, dtype=torch.long)
            inp.x[idx] = rows
            if rows.dtype == torch.bfloat16:
                Xb = O.decode_matrix(rows.view(torch.int16).cpu().numpy().view(np.uint16), True)
            else:
                Xb = O.decode_matrix(rows.cpu().numpy(), False)
        redraws += len(bad)
        still = margin_violations(O.router_logits(xform(Xb), Wr, b), cfg.k, margin)
        bad = [bad[i] for i in still]
        attempt += 1
    return redraws


def make_inputs(cfg, backend: str = "numpy", device=None, margin: float = MARGIN):
    inp = generate(cfg, backend=backend, device=device)
    enforce_margin(inp, margin)
    return inp
