"""CPU checks of the seeded input generators' stated properties (no layer
arithmetic here): the tied-logit inputs that the GPU tie test relies on."""
import numpy as np
import pytest

from moe_synth import MoeConfig, tied_router_inputs


@pytest.mark.parametrize("E,k", [(16, 4), (64, 6), (128, 8), (200, 6)])
def test_tied_inputs_repeat_rows_and_tie_in_the_top_k(E, k):
    cfg = MoeConfig(name="ties", T=5, H=96, I=32, E=E, k=k, seed_index=90)
    r, x = tied_router_inputs(cfg)
    r2, x2 = tied_router_inputs(cfg)
    assert (r == r2).all() and (x == x2).all()                    # seeded
    assert r.dtype == np.float32 and (r == np.round(r)).all() and np.abs(r).max() <= 2
    assert (x == np.round(x)).all() and np.abs(x).max() <= 3
    D = E // 4
    assert all((r[e] == r[e % D]).all() for e in range(E))          # period E/4
    L = x.astype(np.float64) @ r.astype(np.float64).T
    top = -np.sort(-L, axis=1)[:, :k + 1]
    assert (np.diff(top, axis=1) == 0).any(axis=1).all()


def test_tied_inputs_zero_top():
    cfg = MoeConfig(name="ties0", T=7, H=64, I=32, E=48, k=5, seed_index=91)
    r, x = tied_router_inputs(cfg, zero_top=True)
    zero = np.arange(48) % 3 == 1
    assert (r[zero] == 0).all()
    assert (r[~zero][:, 0] == -1).all() and (r[~zero] <= 0).all() and (r[~zero] >= -2).all()
    assert (x >= 1).all() and (x <= 3).all()
    L = x.astype(np.float64) @ r.astype(np.float64).T
    assert (L.max(axis=1) == 0).all()
    assert ((L == 0) == zero[None, :]).all()                       # exactly the zero rows
